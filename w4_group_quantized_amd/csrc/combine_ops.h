// Device helpers of the weighted combine, shared by the combine kernels and
// the launch that fuses a layer's combine with the next layer's router.
#pragma once
#include "common.h"

namespace moe {

constexpr int kMaxK = 32;

// w[j] / (w[0] + ... + w[k-1]) for the k weights in LDS, the sum in that
// order (every thread forms the same sum; the block then meets again so that
// no weight is overwritten while another thread still reads it).
__device__ __forceinline__ void renorm_weights(float *s_w, int k) {
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += s_w[j];
  const float wj = threadIdx.x < (unsigned)k ? s_w[threadIdx.x] / sum : 0.0f;
  __syncthreads();
  if (threadIdx.x < (unsigned)k) s_w[threadIdx.x] = wj;
  __syncthreads();
}

// v[i] += w_j * y_perm[row_j][c + i] for j = 0 .. k-1 in that order, fp32.
// row_of(j) and w_of(j) give the permuted row (in [0, N)) and the weight of
// slot j; eight slots at a time, their row indices first and then all eight
// 16-byte row loads, so that a round costs two memory latencies instead of
// two per slot.  The loads are unconditional (slots past k repeat slot k-1
// and are not added): a load under a branch would make the compiler wait
// for every earlier load at the branch's end.
// init(v) sets the starting values once the first round's loads are out.
struct NoInit {
  __device__ __forceinline__ void operator()(float (&)[8]) const {}
};
template <class RowOf, class WOf, class Init = NoInit>
__device__ __forceinline__ void accumulate_rows(float (&v)[8], const f16 *__restrict__ y_perm,
                                                int H, int c, int k, RowOf row_of, WOf w_of,
                                                Init init = Init()) {
  for (int j0 = 0; j0 < k; j0 += 8) {
    int r[8];
    float wj[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = min(j0 + i, k - 1);
      r[i] = row_of(j);
      wj[i] = w_of(j);
    }
    f16x8 y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = as_f16x8(ld16(y_perm + (size_t)r[i] * H + c));
    if (j0 == 0) init(v);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (j0 + i < k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(wj[i], (float)y[i][e], v[e]);
      }
  }
}

}  // namespace moe
