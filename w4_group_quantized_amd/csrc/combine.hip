// Unpermute + weighted combine with the shared expert, optional RMS norm.
//
// out[t] = y_shared[t] + sum_j w[t][j] * y_perm[inv_pos[t*k + j]] in fp32, in
// that fixed order; the shared expert is always on with weight 1
// (haowenji.com/articles/x-2109226022155796480 §01: 8 routed + 1 shared
// experts per token).  With MOE_RMSNORM the row is divided by
// sqrt(mean(row^2) + eps), as between stacked decode layers.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMaxK = 32;

// One block per token; each thread owns 8-column chunks of the row.
__global__ __launch_bounds__(256) void combine_kernel(const f16 *__restrict__ y_perm,
                                                      const f16 *__restrict__ ys,
                                                      const int32_t *__restrict__ inv_pos,
                                                      const float *__restrict__ w, int k, int H,
                                                      int N, int rmsnorm, float eps,
                                                      f16 *__restrict__ out) {
  __shared__ int s_row[kMaxK];
  __shared__ float s_w[kMaxK];
  __shared__ float s_red[4];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    int r = inv_pos[(size_t)t * k + threadIdx.x];
    s_row[threadIdx.x] = r < 0 ? 0 : (r >= N ? N - 1 : r);
    s_w[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();

  auto row_chunk = [&](int c, float (&v)[8]) {
    if (ys) {
      const f16x8 a = as_f16x8(ld16(ys + (size_t)t * H + c));
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
      const f16x8 y = as_f16x8(ld16(y_perm + (size_t)s_row[j] * H + c));
      const float wj = s_w[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = fmaf(wj, (float)y[i], v[i]);
    }
  };

  float scale = 1.0f;
  if (rmsnorm) {
    float ss = 0.0f;
    for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
      float v[8];
      row_chunk(c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0) s_red[threadIdx.x / kWave] = ss;
    __syncthreads();
    const float tot = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    scale = 1.0f / sqrtf(tot / (float)H + eps);
  }
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float v[8];
    row_chunk(c, v);
    f16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (f16)(v[i] * scale);
    *reinterpret_cast<f16x8 *>(out + (size_t)t * H + c) = o;
  }
}

hipError_t launch_combine(const moe_layer &L, const uint16_t *y_perm, const uint16_t *y_shared,
                          const int32_t *inv_pos, const float *w, int32_t T, uint32_t flags,
                          float eps, uint16_t *out, hipStream_t st) {
  const int k = L.top_k, H = L.hidden;
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, st,
                     reinterpret_cast<const f16 *>(y_perm), reinterpret_cast<const f16 *>(y_shared),
                     inv_pos, w, k, H, T * k, (flags & MOE_RMSNORM) ? 1 : 0, eps,
                     reinterpret_cast<f16 *>(out));
  return hipGetLastError();
}

}  // namespace moe
