// A decode step through stacked layers: the combine (+ RMS norm) of layer i
// and the router, top-k and permutation of layer i + 1 in one launch.
//
// Between stacked layers the output of layer i is the input of layer i + 1
// (haowenji.com/articles/x-2109226022155796480 §01: 42 MoE layers, 8 routed +
// 1 shared experts per token).  Layer i's combine and layer i + 1's router
// each stream almost nothing from HBM and are bound by a few dependent memory
// round trips; run back to back they leave the memory system idle for two
// launches per layer.  Here they share one launch:
//
//   block (token t, expert tile et): forms token t's combined row of layer i
//     exactly as the combine kernels do (the same per-element arithmetic and,
//     with the norm, the same reduction order, so every block of the token
//     holds bitwise the same fp16 row), stores it once (tile 0 does), and
//     computes the logits of layer i + 1's experts of its tile on that fp16
//     row; then it takes a ticket on token t's counter.
//   the last block of token t: softmax + top-k of the token (one wave over
//     its E logits: zwxr.cn/news/276292 §3.2, softmax and top-k fused:
//     lpnh.cn/news/2730718 §2.3); then a ticket on the all-token counter.
//   the last of those: the permutation by expert (xdnf.cn/news/329730 §3.2)
//     of all T*k choices, and the counters are left at zero.
//
// Tiles are dealt to XCDs so that the blocks of one expert tile share an L2:
// block b runs on XCD b % 8 and takes expert tile 8 * ((b / 8) / T) + b % 8.
// Logits and the chosen experts cross XCDs through agent-scope atomic stores
// and loads that read the device coherence point, published before the
// ticket in the way the one-launch router publishes its partial logits.
// Nothing waits on another block: a block that is not last returns.
#include "common.h"
#include "kernels.h"
#include "combine_ops.h"
#include "topk_ops.h"

namespace moe {

constexpr int kStackWaves = 16;      // 1024 threads: 8 columns each up to H = 8192

struct CombineRouteArgs {
  // layer i: combine (+ RMS norm) into out = the input of layer i + 1
  const f16 *y_perm;                // [N, H]
  const f16 *ys;                    // [T, H] or null
  const int32_t *inv_pos_in;        // [T * k], layer i (the same buffer as inv_pos)
  const float *w_in;                // [T * k], layer i (the same buffer as w)
  int N, renorm, norm;
  float eps;
  f16 *out;                         // [T, H]
  // layer i + 1: router, top-k, permutation
  const f16 *wr;                    // [E, H]
  const float *bias;                // [E] or null
  int T, E, H, k;
  int eb;                           // experts per block
  int et;                           // expert tiles, ceil(E / eb)
  float *logits;                    // [T, E] workspace
  unsigned int *tok_counter;        // [T] workspace, zero before and after
  unsigned int *all_counter;        // workspace, zero before and after
  int32_t *idx;                     // [T, k]
  float *w;                         // [T, k]
  int32_t *offsets, *perm_src, *inv_pos;
};

template <int NPER>
__global__ __launch_bounds__(kStackWaves *kWave) void combine_route_kernel(CombineRouteArgs p) {
  __shared__ int s_row[kMaxK];
  __shared__ float s_w[kMaxK];
  __shared__ float s_red[kStackWaves];
  __shared__ u32x4 s_x[8192 / 8];   // the token's fp16 row
  __shared__ int s_idx[kStackMaxT * kMaxK];
  __shared__ int s_cnt[1024];
  __shared__ int s_scan[kStackWaves];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int T = p.T, E = p.E, H = p.H, k = p.k;
  const int xcd = blockIdx.x % 8, i = blockIdx.x / 8;
  const int t = i % T;
  const int et = (i / T) * 8 + xcd;
  if (et >= p.et) return;           // grid padding: takes no ticket

  // ---- the combined row of token t (the arithmetic of combine_norm_kernel
  // and, without the norm, of combine_cols_kernel, element for element)
  if (tid < k) {
    const int r = p.inv_pos_in[(size_t)t * k + tid];
    s_row[tid] = r < 0 ? 0 : (r >= p.N ? p.N - 1 : r);
    s_w[tid] = p.w_in[(size_t)t * k + tid];
  }
  const int c = tid * 8;
  const bool live = c < H;
  const bool wave_live = __ballot(live) != 0ull;   // wave-uniform
  f16x8 ysv = {};
  if (p.ys && live) ysv = as_f16x8(ld16(p.ys + (size_t)t * H + c));

  // The router rows do not depend on the combine: the first 512 chunks (8
  // per lane) of the wave's first two experts are loaded as soon as the
  // combine's own row loads are out (a CU serves its loads in issue order,
  // and the block's router rows, 144 KB at 16 tokens, would otherwise hold
  // the combine's loads back).  Wave w takes experts e0 + w, e0 + w + 16,
  // ...; lane l the
  // 8-column chunks l, l + 64, ... of the row (each load instruction reads
  // 1 KB of a router row).
  const int e0 = et * p.eb, e_end = min(e0 + p.eb, E);
  const int nch = H / 8;
  const rsrc_t wrs = make_rsrc(p.wr, (uint32_t)E * (uint32_t)H * 2u);
  auto load_w = [&](int e, int ch0, u32x4 (&wv)[8]) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ch = ch0 + u * kWave + lane;
      wv[u] = bload16(wrs, e < e_end && ch < nch ? ((uint32_t)e * H + (uint32_t)ch * 8u) * 2u
                                                 : 0xFFFFFFF0u, 0);
    }
  };
  u32x4 wa[8], wb[8];
  auto prefetch_w = [&] {
    load_w(e0 + wid, 0, wa);
    load_w(e0 + wid + kStackWaves, 0, wb);
  };

  float v[8];
  __syncthreads();
  if (p.renorm) renorm_weights(s_w, k);
  if (live) {
    accumulate_rows(v, p.y_perm, H, c, k, [&](int j) { return s_row[j]; },
                    [&](int j) { return s_w[j]; }, [&](float (&a)[8]) {
                      prefetch_w();
#pragma unroll
                      for (int j = 0; j < 8; ++j) a[j] = (float)ysv[j];
                    });
  } else {
    // lanes past the row: a wave with some live lanes loads with them; a
    // wave with none loads its rows after the combine, so that its loads do
    // not queue ahead of the combine's in the CU
    if (wave_live) prefetch_w();
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }
  float scale = 1.0f;
  if (p.norm) {
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
    ss = wave_sum(ss);
    if (lane == 0) s_red[wid] = ss;
    __syncthreads();
    // the waves past the row hold 0 and add nothing: the same sum as the
    // combine kernel's over its ceil(H / 512) waves
    float tot = 0.0f;
    for (int j = 0; j < kStackWaves; ++j) tot += s_red[j];
    scale = 1.0f / sqrtf(tot / (float)H + p.eps);
  }
  if (live) {
    f16x8 o;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (f16)(v[j] * scale);
    s_x[tid] = __builtin_bit_cast(u32x4, o);
    if (et == 0) *reinterpret_cast<f16x8 *>(p.out + (size_t)t * H + c) = o;
  }
  __syncthreads();

  // ---- logits of the tile's experts on the fp16 row: per lane its chunks in
  // order, then across the wave
  {
    auto dot = [&](const u32x4 (&wv)[8], int ch0, float a) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ch = ch0 + u * kWave + lane;
        if (ch < nch) {
          const f16x8 xw = as_f16x8(s_x[ch]);
          const f16x8 ww = as_f16x8(wv[u]);
#pragma unroll
          for (int j = 0; j < 8; ++j) a = fmaf((float)xw[j], (float)ww[j], a);
        }
      }
      return a;
    };
    auto finish = [&](int e, int ch_from, float a) {   // remaining chunks, wave sum, store
      for (int ch0 = ch_from; ch0 < nch; ch0 += 8 * kWave) {
        u32x4 wv[8];
        load_w(e, ch0, wv);
        a = dot(wv, ch0, a);
      }
      a = wave_sum(a);
      if (lane == 0) {
        if (p.bias) a += p.bias[e];
        // written through to the device coherence point (no L2 flush)
        __hip_atomic_store(&p.logits[(size_t)t * E + e], a, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    const int ea = e0 + wid, eb = ea + kStackWaves;
    if (!wave_live) {
      load_w(ea, 0, wa);
      load_w(eb, 0, wb);
    }
    if (ea < e_end) finish(ea, 8 * kWave, dot(wa, 0, 0.0f));
    if (eb < e_end) finish(eb, 8 * kWave, dot(wb, 0, 0.0f));
    for (int e = eb + kStackWaves; e < e_end; e += kStackWaves) finish(e, 0, 0.0f);
  }

  // ---- ticket of token t: this block's stores complete before the barrier,
  // the barrier before the increment (the one-launch router's handoff)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&p.tok_counter[t], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == (unsigned)p.et - 1u;
  __syncthreads();
  if (!s_last) return;

  // ---- the token's last block: softmax + top-k over its E logits
  if (tid == 0)
    __hip_atomic_store(&p.tok_counter[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (wid == 0) {
    const rsrc_t lrs = make_rsrc(p.logits + (size_t)t * E, (uint32_t)E * 4u);
    wave_softmax_topk<NPER>(
        [&](int e) {
          return __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(lrs, (uint32_t)e * 4u, 0, kBufCoherent));
        },
        E, k,
        [&](int j, int e, float pr) {
          __hip_atomic_store(&p.idx[(size_t)t * k + j], e, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
          p.w[(size_t)t * k + j] = pr;
          s_idx[j] = e;
        });
    // one token: this is the last block of all, and the permutation is the
    // order of its k choices (no second ticket, no reload of the choices)
    if (T == 1) one_token_permutation(s_idx, k, E, p.offsets, p.perm_src, p.inv_pos);
  }
  if (T == 1) return;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(p.all_counter, 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == (unsigned)T - 1u;
  __syncthreads();
  if (!s_last) return;

  // ---- the last token's block: the permutation of all T * k choices
  if (tid == 0)
    __hip_atomic_store(p.all_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int N = T * k;
  const rsrc_t irs = make_rsrc(p.idx, (uint32_t)N * 4u);
  for (int f = tid; f < N; f += blockDim.x) {
    const int e = (int)__builtin_amdgcn_raw_buffer_load_b32(irs, (uint32_t)f * 4u, 0, kBufCoherent);
    s_idx[f] = e < 0 ? 0 : (e >= E ? E - 1 : e);
  }
  static_assert(kStackWaves * kWave >= 1024, "one thread per expert in the permutation's scan");
  build_permutation(s_idx, N, E, s_cnt, s_scan, p.offsets, p.perm_src, p.inv_pos);
}

// Experts per block: as many tiles as give every CU one block (32 CUs per
// XCD, T blocks per tile), each CU then loading the fewest router rows.
static int stack_experts_per_block(int T, int E) {
  const int tiles = 8 * (T < 32 ? 32 / T : 1);
  return (E + tiles - 1) / tiles;
}

bool stack_fused(const moe_layer &L, int32_t T) {
  return T >= 1 && T <= kStackMaxT && L.hidden <= 8192 && L.top_k <= kMaxK;
}

hipError_t launch_combine_route(const moe_layer &cur, const moe_layer &next,
                                const uint16_t *y_perm, const uint16_t *y_shared,
                                int32_t *inv_pos, float *topk_w, int32_t T, uint32_t flags,
                                float eps, uint16_t *out, int32_t *topk_idx, int32_t *offsets,
                                int32_t *perm_src, float *logits, unsigned int *sync,
                                hipStream_t st) {
  CombineRouteArgs a{};
  a.y_perm = reinterpret_cast<const f16 *>(y_perm);
  a.ys = reinterpret_cast<const f16 *>(y_shared);
  a.inv_pos_in = inv_pos;
  a.w_in = topk_w;
  a.N = T * cur.top_k;
  a.renorm = (flags & MOE_RENORM) ? 1 : 0;
  a.norm = (flags & MOE_RMSNORM) ? 1 : 0;
  a.eps = eps;
  a.out = reinterpret_cast<f16 *>(out);
  a.wr = reinterpret_cast<const f16 *>(next.router_w);
  a.bias = next.router_b;
  a.T = T; a.E = next.num_experts; a.H = next.hidden; a.k = next.top_k;
  a.eb = stack_experts_per_block(T, a.E);
  a.et = (a.E + a.eb - 1) / a.eb;
  a.logits = logits;
  a.tok_counter = sync + kStackTokCounter;
  a.all_counter = sync + kStackAllCounter;
  a.idx = topk_idx; a.w = topk_w;
  a.offsets = offsets; a.perm_src = perm_src; a.inv_pos = inv_pos;
  const int blocks = 8 * T * ((a.et + 7) / 8);
#define MOE_STACK_LAUNCH(n)                                                                     \
  hipLaunchKernelGGL(combine_route_kernel<n>, dim3(blocks), dim3(kStackWaves * kWave), 0, st, \
                     a)
  MOE_NPER_SWITCH(a.E, MOE_STACK_LAUNCH)
#undef MOE_STACK_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
