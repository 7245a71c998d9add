// Router: logits on the matrix cores, softmax + top-k fused with wavefront
// reductions, and (for decode-sized batches) the permutation by expert in the
// same launch.
//
// Softmax over the expert logits followed by a descending partial sort for
// the first k: zwxr.cn/news/276292 §3.2 (routing engine).  Softmax and top-k
// fused into one kernel so the probabilities never round-trip through global
// memory: lpnh.cn/news/2730718 §2.3.  Tokens grouped by expert for one grouped
// GEMM: xdnf.cn/news/329730 §3.2.  Ties go to the lower expert index; the
// combine weights are the softmax probabilities of the chosen experts, not
// renormalised.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "tiles.h"
#include "topk_ops.h"

namespace moe {

// ------------------------------------------------------------ any batch size
// logits[t][e] = x[t] . Wr[e] + b[e].  One block per (16-token tile,
// 16-expert tile); its 4 waves split K and their partial sums are added in a
// fixed order.
__global__ __launch_bounds__(256) void router_logits_kernel(const f16 *__restrict__ x,
                                                            const f16 *__restrict__ wr,
                                                            const float *__restrict__ bias,
                                                            int T, int E, int H,
                                                            float *__restrict__ logits) {
  __shared__ float red[3 * 4 * kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int r = lane & 15, kb = lane >> 4;
  const int etiles = (E + 15) / 16;
  const int mt = blockIdx.x / etiles, et = blockIdx.x % etiles;
  const int tok0 = mt * 16;
  const int rows = min(16, T - tok0);
  const ARows arow(x + (size_t)tok0 * H, rows, H, r, r < rows, kb);   // surplus rows read zeros
  const int e = et * 16 + r;
  const f16 *wrow[1] = {wr + (size_t)min(e, E - 1) * H};
  f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
  const int G = H / kGroup;
  f16_tiles<1>(arow, wrow, kb, wid * G / 4, (wid + 1) * G / 4, acc);
  ksplit_reduce<1>(acc, red);
  if (wid != 0 || e >= E) return;
  const float b = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = 4 * kb + j;
    if (tok < rows) logits[(size_t)(tok0 + tok) * E + e] = acc[0][j] + b;
  }
}

// Prefill-sized batches: one block per 32 tokens x 128 experts, so x is
// read from memory once instead of once per 16-expert tile.  K is walked in
// chunks of 128 columns.  The block loads each chunk's 32 token rows (8 KB)
// and 128 router rows (32 KB) as coalesced 16-byte pieces (consecutive
// threads cover consecutive pieces of a row), kRouterPf chunks ahead in
// registers, and stores them into one of two LDS stages; wave w multiplies
// the 32 tokens by experts 32w .. 32w+31 from LDS with
// v_mfma_f32_32x32x16_f16.  Each LDS row is padded by one piece, so the
// operand reads of 16 consecutive rows fall on distinct banks.  In each
// 64-column block, lane (row l%32, half l/32) supplies pieces 4*(l/32) + s
// to MFMA s (k = 8s .. 8s+7 and 32+8s .. 32+8s+7); the four accumulators
// (one per s) are summed in a fixed order at the end.
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kRouterKc = 2;   // 64-column K blocks per chunk
constexpr int kRouterPf = 2;   // chunks in flight in registers ahead of the LDS stage
constexpr int kRouterRow = 8 * kRouterKc + 1;   // LDS row stride in 16-byte pieces (+1 pad)

__global__ __launch_bounds__(256) void router_logits_wide_kernel(const f16 *__restrict__ x,
                                                                 const f16 *__restrict__ wr,
                                                                 const float *__restrict__ bias,
                                                                 int T, int E, int H,
                                                                 float *__restrict__ logits) {
  constexpr int KC = kRouterKc, PPR = 8 * KC;   // pieces per row and chunk
  __shared__ u32x4 sx[2][32 * kRouterRow];
  __shared__ u32x4 sw[2][128 * kRouterRow];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int etiles = (E + 127) / 128;
  const int tok0 = (blockIdx.x / etiles) * 32;
  const int eb = (blockIdx.x % etiles) * 128;
  const int l32 = lane & 31, kh = lane >> 5;
  const int C = H / (64 * KC);
  // this thread's pieces: x piece tid + 256j (j < KC), router piece tid + 256j
  // (j < 4KC); piece p is row p / PPR, column piece p % PPR
  const f16 *xp[KC];
  const f16 *wp[4 * KC];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int p = tid + 256 * j;
    xp[j] = x + (size_t)min(tok0 + p / PPR, T - 1) * H + (p % PPR) * 8;
  }
#pragma unroll
  for (int j = 0; j < 4 * KC; ++j) {
    const int p = tid + 256 * j;
    wp[j] = wr + (size_t)min(eb + p / PPR, E - 1) * H + (p % PPR) * 8;
  }
  struct Pieces {
    u32x4 x[KC], w[4 * KC];
  };
  auto gload = [&](Pieces &pc, int ci) {
    const size_t k = (size_t)min(ci, C - 1) * 64 * KC;
#pragma unroll
    for (int j = 0; j < KC; ++j) pc.x[j] = ld16(xp[j] + k);
#pragma unroll
    for (int j = 0; j < 4 * KC; ++j) pc.w[j] = ld16(wp[j] + k);
  };
  auto lstore = [&](const Pieces &pc, int st) {
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const int p = tid + 256 * j;
      sx[st][(p / PPR) * kRouterRow + p % PPR] = pc.x[j];
    }
#pragma unroll
    for (int j = 0; j < 4 * KC; ++j) {
      const int p = tid + 256 * j;
      sw[st][(p / PPR) * kRouterRow + p % PPR] = pc.w[j];
    }
  };
  f32x16 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = (f32x16){};
  auto compute = [&](int st) {
#pragma unroll
    for (int h = 0; h < KC; ++h)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = sx[st][l32 * kRouterRow + 8 * h + 4 * kh + s];
        const u32x4 b = sw[st][(wv * 32 + l32) * kRouterRow + 8 * h + 4 * kh + s];
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a), as_f16x8(b), acc[s], 0, 0, 0);
      }
  };
  constexpr int PF = kRouterPf;
  Pieces r[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) gload(r[u], u);
  lstore(r[0], 0);
  gload(r[0], PF);
  __syncthreads();
  for (int c0 = 0;; c0 += PF) {
    bool done = false;
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      if (!done) {
        const int ci = c0 + u;
        compute(ci & 1);
        if (ci + 1 < C) {
          lstore(r[(u + 1) % PF], (ci + 1) & 1);
          gload(r[(u + 1) % PF], ci + 1 + PF);
        }
        __syncthreads();
        done = ci + 1 >= C;
      }
    }
    if (done) break;
  }
  const int e = eb + wv * 32 + l32;
  if (e >= E) return;
  const float bb = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int tok = tok0 + 8 * (q >> 2) + 4 * kh + (q & 3);
    if (tok < T) logits[(size_t)tok * E + e] = ((acc[0][q] + acc[1][q]) + (acc[2][q] + acc[3][q])) + bb;
  }
}

// One wave per token, 4 tokens per block.
template <int NPER>
__global__ __launch_bounds__(256) void softmax_topk_kernel(const float *__restrict__ logits,
                                                           int T, int E, int k,
                                                           int32_t *__restrict__ idx,
                                                           float *__restrict__ w) {
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const float *lt = logits + (size_t)t * E;
  wave_softmax_topk<NPER>([&](int e) { return lt[e]; }, E, k, [&](int j, int e, float pr) {
    idx[(size_t)t * k + j] = e;
    w[(size_t)t * k + j] = pr;
  });
}

// ------------------------------------------------------------ decode batches
// Route and permute in one launch.  Blocks (16-token tile, 16-expert tile,
// K part) write partial logits; the last block to finish (device-wide
// counter) adds the partials in K-part order plus the bias, runs softmax and
// top-k (one wave per token), then builds the per-expert segments in LDS:
// histogram, exclusive scan, and stable ranks by ballot-matching expert ids
// 64 entries at a time.  It then resets the counter to 0.
constexpr int kFusedWaves = 16;

struct FusedRouteArgs {
  const f16 *x;
  const f16 *wr;
  const float *bias;
  int T, E, H, k, ksb;           // ksb: K parts across blocks
  float *partial;                // [ksb, T, E]
  unsigned int *counter;         // zero before the launch, zero after
  int32_t *idx;                  // [T, k]
  float *w;                      // [T, k]
  int32_t *offsets;              // [E + 1]
  int32_t *perm_src;             // [T*k]
  int32_t *inv_pos;              // [T*k]
};

template <int NPER>
__global__ __launch_bounds__(kFusedWaves * kWave) void route_permute_kernel(FusedRouteArgs p) {
  __shared__ float red[(kFusedWaves - 1) * 4 * kWave];
  __shared__ int s_idx[kFusedMaxT * 32];
  __shared__ float s_logit[kFusedMaxLogits];
  __shared__ int s_cnt[1024];
  __shared__ int s_scan[kFusedWaves];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int r = lane & 15, kb = lane >> 4;
  const int T = p.T, E = p.E, H = p.H, k = p.k;
  const int G = H / kGroup;
  const int TE = T * E, TEp = (TE + 3) & ~3;   // logits per K part, padded

  // ---- partial logits of this block's (token tile, expert tile, K part)
  {
    const int etiles = (E + 15) / 16;
    const int kp = blockIdx.x % p.ksb;
    const int et = (blockIdx.x / p.ksb) % etiles;
    const int mt = blockIdx.x / (p.ksb * etiles);
    const int tok0 = mt * 16;
    const int rows = min(16, T - tok0);
    const ARows arow(p.x + (size_t)tok0 * H, rows, H, r, r < rows, kb);
    const int e = et * 16 + r;
    const f16 *wrow[1] = {p.wr + (size_t)min(e, E - 1) * H};
    const int kg0 = kp * G / p.ksb, kg1 = (kp + 1) * G / p.ksb;
    const int n = kg1 - kg0;
    f32x4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
    f16_tiles<1>(arow, wrow, kb, kg0 + wid * n / kFusedWaves, kg0 + (wid + 1) * n / kFusedWaves,
                 acc);
    ksplit_reduce<1, kFusedWaves>(acc, red);
    if (wid == 0 && e < E) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = 4 * kb + j;
        if (tok < rows)   // written through to the device coherence point (no L2 flush)
          __hip_atomic_store(&p.partial[(size_t)kp * TEp + (size_t)(tok0 + tok) * E + e], acc[0][j],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  // ---- the last block continues.  The partials travel as agent-scope
  // atomic stores and loads, which reach / read the device coherence point
  // directly; waiting for this wave's stores to complete before the barrier
  // orders them before the counter increment, so no L2 write-back or
  // invalidate (what a full device fence costs across the XCDs) is needed.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(p.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;

  // logits = sum of the K parts in order + bias, into LDS; every thread's
  // loads are independent so they are all in flight together
  {
    // four logits per thread and K part: 16-byte loads that read the device
    // coherence point (sc1), like the agent-scope atomic loads they replace.
    // The loads are unconditional, so none of them waits for another:
    // vectors past the last logit read in-bounds values that are never
    // stored.  The bias (a zero-length buffer when there is none) is loaded
    // in the same round.
    const rsrc_t prs = make_rsrc(p.partial, (uint32_t)(p.ksb * TEp) * 4u);
    const rsrc_t brs = make_rsrc(p.bias, p.bias ? (uint32_t)E * 4u : 0u);
    auto sum_parts = [&](auto nparts_tag, auto nvec_tag) {
      constexpr int NP = decltype(nparts_tag)::value;   // K parts held at once
      constexpr int NV = decltype(nvec_tag)::value;     // vectors per thread at once
      for (int base = 0; base < TEp / 4; base += NV * kFusedWaves * kWave) {
        f32x4 part[NV][NP];
        float bv[NV][4];
#pragma unroll
        for (int u = 0; u < NV; ++u) {   // every load of the round before any sum
          const int i4 = base + tid + u * kFusedWaves * kWave;
#pragma unroll
          for (int kp = 0; kp < NP; ++kp)
            part[u][kp] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           prs, (uint32_t)(kp * TEp + 4 * i4) * 4u, 0, kBufCoherent));
#pragma unroll
          for (int c = 0; c < 4; ++c)
            bv[u][c] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(
                           brs, (uint32_t)(min(4 * i4 + c, TE - 1) % E) * 4u, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < NV; ++u) {
          const int i4 = base + tid + u * kFusedWaves * kWave;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int i = 4 * i4 + c;
            if (i < TE) {
              float a = part[u][0][c];
#pragma unroll
              for (int kp = 1; kp < NP; ++kp) a += part[u][kp][c];
              s_logit[i] = a + bv[u][c];
            }
          }
        }
      }
    };
    // ksb is a power of two up to kFusedMaxKsb: one instantiation per value,
    // so every load issued is a part that exists; up to 4 parts, two vectors
    // per thread (8192 logits in one round trip)
    using std::integral_constant;
    static_assert(kFusedMaxKsb == 16, "one case per power of two up to kFusedMaxKsb");
    switch (p.ksb) {
      case 1: sum_parts(integral_constant<int, 1>(), integral_constant<int, 2>()); break;
      case 2: sum_parts(integral_constant<int, 2>(), integral_constant<int, 2>()); break;
      case 4: sum_parts(integral_constant<int, 4>(), integral_constant<int, 2>()); break;
      case 8: sum_parts(integral_constant<int, 8>(), integral_constant<int, 1>()); break;
      default: sum_parts(integral_constant<int, kFusedMaxKsb>(), integral_constant<int, 1>());
    }
  }
  __syncthreads();

  // softmax + top-k, one wave per token
  for (int t = wid; t < T; t += kFusedWaves) {
    const float *lt = s_logit + t * E;
    wave_softmax_topk<NPER>([&](int e) { return lt[e]; }, E, k, [&](int j, int e, float pr) {
      p.idx[(size_t)t * k + j] = e;
      p.w[(size_t)t * k + j] = pr;
      s_idx[t * k + j] = e;
    });
  }
  static_assert(kFusedWaves * kWave >= 1024, "one thread per expert in the permutation's scan");
  build_permutation(s_idx, T * k, E, s_cnt, s_scan, p.offsets, p.perm_src, p.inv_pos);
  if (tid == 0) __hip_atomic_store(p.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// K parts across blocks: only when there are too few expert tiles to spread
// the router weights over enough CUs (each part is one more partial per
// logit for the last block to add after the cross-XCD fence).
int fused_route_ksb(const moe_layer &L) {
  const int G = L.hidden / kGroup;
  const int etiles = (L.num_experts + 15) / 16;
  int ksb = 1;
  while (ksb < kFusedMaxKsb && etiles * ksb < 64 && G / (2 * ksb) >= 8) ksb *= 2;
  return ksb;
}

hipError_t launch_route(const moe_layer &L, const uint16_t *x, int32_t T, int32_t *idx,
                        float *w, float *logits, hipStream_t st) {
  const int E = L.num_experts, H = L.hidden;
  if (T >= kRouterWideMinT) {
    const int blocks = ((T + 31) / 32) * ((E + 127) / 128);
    hipLaunchKernelGGL(router_logits_wide_kernel, dim3(blocks), dim3(256), 0, st,
                       reinterpret_cast<const f16 *>(x),
                       reinterpret_cast<const f16 *>(L.router_w), L.router_b, T, E, H, logits);
  } else {
    const int blocks = ((T + 15) / 16) * ((E + 15) / 16);
    hipLaunchKernelGGL(router_logits_kernel, dim3(blocks), dim3(256), 0, st,
                       reinterpret_cast<const f16 *>(x),
                       reinterpret_cast<const f16 *>(L.router_w), L.router_b, T, E, H, logits);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
#define MOE_TOPK_LAUNCH(n)                                                             \
  hipLaunchKernelGGL(softmax_topk_kernel<n>, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, \
                     E, L.top_k, idx, w)
  MOE_NPER_SWITCH(E, MOE_TOPK_LAUNCH)
#undef MOE_TOPK_LAUNCH
  return hipGetLastError();
}

hipError_t launch_route_permute_fused(const moe_layer &L, const uint16_t *x, int32_t T,
                                      int32_t *idx, float *w, int32_t *offsets,
                                      int32_t *perm_src, int32_t *inv_pos, float *partial,
                                      unsigned int *counter, hipStream_t st) {
  FusedRouteArgs a{};
  a.x = reinterpret_cast<const f16 *>(x);
  a.wr = reinterpret_cast<const f16 *>(L.router_w);
  a.bias = L.router_b;
  a.T = T; a.E = L.num_experts; a.H = L.hidden; a.k = L.top_k;
  a.ksb = fused_route_ksb(L);
  a.partial = partial; a.counter = counter;
  a.idx = idx; a.w = w; a.offsets = offsets; a.perm_src = perm_src; a.inv_pos = inv_pos;
  const int blocks = ((T + 15) / 16) * ((a.E + 15) / 16) * a.ksb;
#define MOE_FUSED_LAUNCH(n) \
  hipLaunchKernelGGL(route_permute_kernel<n>, dim3(blocks), dim3(kFusedWaves * kWave), 0, st, a)
  MOE_NPER_SWITCH(a.E, MOE_FUSED_LAUNCH)
#undef MOE_FUSED_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
