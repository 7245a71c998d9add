// Router: logits on the matrix cores, then softmax and top-k fused in one
// kernel with wavefront reductions.
//
// Softmax over the expert logits followed by a descending partial sort for
// the first k: zwxr.cn/news/276292 §3.2 (routing engine).  Softmax and top-k
// fused into one kernel so the probabilities never round-trip through global
// memory: lpnh.cn/news/2730718 §2.3.  Ties go to the lower expert index; the
// combine weights are the softmax probabilities of the chosen experts, not
// renormalised.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

namespace moe {

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
  const f16 *arow = x + (size_t)(tok0 + min(r, rows - 1)) * H;   // surplus rows: duplicates, dropped
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

// Ranking key: numbers above NaN, NaN above empty slots; among equals the
// lower expert index first.
struct Cand {
  float v;
  int cls;   // 2 = number, 1 = NaN, 0 = empty / already chosen
  int e;
};

__device__ __forceinline__ bool better(const Cand &a, const Cand &b) {
  if (a.cls != b.cls) return a.cls > b.cls;
  if (a.cls == 2 && a.v != b.v) return a.v > b.v;
  return a.e < b.e;
}

__device__ __forceinline__ float max_nan(float a, float b) {
  return (a != a || b != b) ? __builtin_nanf("") : fmaxf(a, b);
}

constexpr int kMaxPerLane = 16;   // E <= 1024

// One wave per token: softmax over E logits, then k rounds of a wave-wide
// arg-max.  4 tokens per 256-thread block.
__global__ __launch_bounds__(256) void softmax_topk_kernel(const float *__restrict__ logits,
                                                           int T, int E, int k,
                                                           int32_t *__restrict__ idx,
                                                           float *__restrict__ w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const float *lt = logits + (size_t)t * E;
  float v[kMaxPerLane];
  float m = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    v[i] = e < E ? lt[e] : -__builtin_inff();
    if (e < E) m = max_nan(m, v[i]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max_nan(m, __shfl_xor(m, o, kWave));
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i)
    if (lane + i * kWave < E) s += expf(v[i] - m);
  s = wave_sum(s);
  uint32_t taken = 0;   // bit i: entry i of this lane already chosen
  for (int j = 0; j < k; ++j) {
    Cand best{0.0f, 0, 0x7fffffff};
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (e < E && !((taken >> i) & 1u)) {
        Cand c{v[i], v[i] != v[i] ? 1 : 2, e};
        if (better(c, best)) best = c;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      Cand other{__shfl_xor(best.v, o, kWave), __shfl_xor(best.cls, o, kWave),
                 __shfl_xor(best.e, o, kWave)};
      if (better(other, best)) best = other;
    }
    if ((best.e & (kWave - 1)) == lane) taken |= 1u << (best.e / kWave);
    if (lane == 0) {
      idx[(size_t)t * k + j] = best.e;
      w[(size_t)t * k + j] = expf(best.v - m) / s;
    }
  }
}

hipError_t launch_route(const moe_layer &L, const uint16_t *x, int32_t T, int32_t *idx,
                        float *w, float *logits, hipStream_t st) {
  const int E = L.num_experts, H = L.hidden;
  const int blocks = ((T + 15) / 16) * ((E + 15) / 16);
  hipLaunchKernelGGL(router_logits_kernel, dim3(blocks), dim3(256), 0, st,
                     reinterpret_cast<const f16 *>(x),
                     reinterpret_cast<const f16 *>(L.router_w), L.router_b, T, E, H, logits);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(softmax_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, st, logits, T, E,
                     L.top_k, idx, w);
  return hipGetLastError();
}

}  // namespace moe
