// Softmax + top-k of one token on one wave, and the permutation of the
// chosen (token, slot) entries by expert: the device code shared by the
// router launches and by the launch that fuses a layer's combine with the
// next layer's router.
//
// Softmax over the expert logits followed by a descending partial sort for
// the first k: zwxr.cn/news/276292 §3.2 (routing engine).  Tokens grouped by
// expert for one grouped GEMM: xdnf.cn/news/329730 §3.2.  Ties go to the
// lower expert index.
#pragma once
#include "common.h"

namespace moe {

// One wave: softmax over the E logits of one token and its k best experts in
// order.  get_expert(e) returns the logit of expert e; lane l holds experts
// l + 64 i (i < NPER), read unconditionally (past E: expert E-1, then
// masked) so that all NPER reads are in flight together.  Each lane sorts
// its NPER (logit, expert) keys once; every round is one wave-wide maximum
// over the lanes' current heads, and the winning lane shifts its list.
// Lane j < k hands the j-th choice to store(j, expert, probability); its
// logit comes back out of the winning key (no second read of the logits).
template <int NPER, class GetE, class Store>
__device__ __forceinline__ void wave_softmax_topk(GetE get_expert, int E, int k, Store store) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[NPER];
  uint64_t key[NPER];
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < NPER; ++i) v[i] = get_expert(min(lane + i * kWave, E - 1));
#pragma unroll
  for (int i = 0; i < NPER; ++i) {
    const int e = lane + i * kWave;
    v[i] = e < E ? v[i] : -__builtin_inff();
    key[i] = e < E ? route_key(v[i], e) : 0ull;
    if (e < E) m = fmax_nan(m, v[i]);
  }
  m = wave_max_nan_dpp(m);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NPER; ++i)
    if (lane + i * kWave < E) s += expf(v[i] - m);
  s = wave_sum_dpp(s);
  // sort this lane's keys, descending (odd-even transposition network)
#pragma unroll
  for (int pass = 0; pass < NPER; ++pass)
#pragma unroll
    for (int i = pass & 1; i + 1 < NPER; i += 2)
      if (key[i + 1] > key[i]) {
        const uint64_t t = key[i]; key[i] = key[i + 1]; key[i + 1] = t;
      }
  // k rounds; the winner of round j is uniform, lane j records it.  The
  // winner is the largest head key: its value-order word alone decides
  // unless several heads share it (equal logits, NaN or empty heads), and
  // then the full 64-bit comparison does.
  uint64_t mine = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t hi = (uint32_t)(key[0] >> 32);
    const uint32_t mhi = wave_max_u32(hi);
    const uint64_t tied = __ballot(hi == mhi);
    uint64_t best;
    if (__popcll(tied) == 1) {   // wave-uniform
      const int owner = __ffsll((long long)tied) - 1;
      best = ((uint64_t)mhi << 32) | (uint32_t)__builtin_amdgcn_readlane((uint32_t)key[0], owner);
    } else {
      best = wave_max_u64(key[0]);
    }
    if (lane == j) mine = best;
    if (key[0] == best) {   // the owner lane: its head won, shift its list
#pragma unroll
      for (int i = 0; i + 1 < NPER; ++i) key[i] = key[i + 1];
      key[NPER - 1] = 0ull;
    }
  }
  if (lane < k)            // the k weights in parallel
    store(lane, route_key_expert(mine), expf(route_key_value(mine) - m) / s);
}

// The permutation of one token's k choices (distinct experts, in s_idx[0..k),
// k <= 64): their order by expert.  One wave; the same offsets, perm_src and
// inv_pos as build_permutation gives for these k entries.
__device__ __forceinline__ void one_token_permutation(const int *s_idx, int k, int E,
                                                      int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ perm_src,
                                                      int32_t *__restrict__ inv_pos) {
  const int lane = threadIdx.x & (kWave - 1);
  const int mine = lane < k ? s_idx[lane] : E;
  int rank = 0;
  for (int i = 0; i < k; ++i) rank += __builtin_amdgcn_readlane(mine, i) < mine ? 1 : 0;
  if (lane < k) {
    perm_src[rank] = lane;
    inv_pos[lane] = rank;
  }
  for (int e = lane; e <= E; e += kWave) {   // offsets[e] = choices below expert e
    int c = 0;
    for (int i = 0; i < k; ++i) c += __builtin_amdgcn_readlane(mine, i) < e ? 1 : 0;
    offsets[e] = c;
  }
}

// The kernels that run it are instantiated per number of logits per lane
// (NPER = ceil(E / 64), 1..16 for E <= 1024) and the host launches the one
// that fits: a kernel holding all sixteen variants behind a switch measured
// 1.6 us slower per call at 8 tokens (its cold tail runs once per launch).
#define MOE_NPER_SWITCH(E, CASE)                                            \
  switch (((E) + kWave - 1) / kWave) {                                      \
    case 1: CASE(1); break;   case 2: CASE(2); break;                       \
    case 3: CASE(3); break;   case 4: CASE(4); break;                       \
    case 5: CASE(5); break;   case 6: CASE(6); break;                       \
    case 7: CASE(7); break;   case 8: CASE(8); break;                       \
    case 9: CASE(9); break;   case 10: CASE(10); break;                     \
    case 11: CASE(11); break; case 12: CASE(12); break;                     \
    case 13: CASE(13); break; case 14: CASE(14); break;                     \
    case 15: CASE(15); break; default: CASE(16); break;                     \
  }

// The permutation of N = T*k (token, slot) entries whose experts are in LDS
// (s_idx[f] for flat index f): per-expert counts, their exclusive scan into
// offsets[0..E], and the stable scatter (perm_src, inv_pos).  Block-wide;
// needs blockDim.x >= E (one thread per expert in the scan), s_cnt holding E
// ints and s_scan one int per wave.
__device__ __forceinline__ void build_permutation(const int *s_idx, int N, int E, int *s_cnt,
                                                  int *s_scan, int32_t *__restrict__ offsets,
                                                  int32_t *__restrict__ perm_src,
                                                  int32_t *__restrict__ inv_pos) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  for (int e = tid; e < E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();

  // histogram and exclusive scan -> offsets
  for (int f = tid; f < N; f += blockDim.x) atomicAdd(&s_cnt[s_idx[f]], 1);
  __syncthreads();
  const int cnt = tid < E ? s_cnt[tid] : 0;
  int total;
  const int run = block_excl_scan(cnt, s_scan, &total);
  __syncthreads();   // every s_cnt read is done before it is overwritten
  if (tid < E) {
    offsets[tid] = run;
    s_cnt[tid] = run;   // running next-row counter of segment e
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();

  // stable ranks: wave 0 walks the flat entries in order, 64 at a time
  if (wid == 0) {
    const uint64_t below = (1ull << lane) - 1ull;
    for (int base = 0; base < N; base += kWave) {
      const int f = base + lane;
      const bool valid = f < N;
      const int e = valid ? s_idx[f] : E;   // E marks an empty lane
      uint64_t same = ~0ull;
#pragma unroll
      for (int b = 0; b < 11; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
      }
      const int rank = __popcll(same & below);
      const int start = valid ? s_cnt[e] : 0;
      if (valid && (same & below) == 0ull) s_cnt[e] = start + __popcll(same);
      if (valid) {
        perm_src[start + rank] = f;
        inv_pos[f] = start + rank;
      }
    }
  }
}

}  // namespace moe
