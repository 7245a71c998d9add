// Unpermute + weighted combine with the shared expert, optional RMS norm.
//
// out[t] = y_shared[t] + sum_j w[t][j] * y_perm[inv_pos[t*k + j]] in fp32, in
// that fixed order; the shared expert is always on with weight 1
// (haowenji.com/articles/x-2109226022155796480 §01: 8 routed + 1 shared
// experts per token).  With MOE_RENORM each w[t][j] is first divided by
// w[t][0] + ... + w[t][k-1] (summed in that order).  With MOE_RMSNORM the row
// is divided by sqrt(mean(row^2) + eps), as between stacked decode layers.
#include "common.h"
#include "kernels.h"
#include "combine_ops.h"

namespace moe {

// One block per token; each thread owns 8-column chunks of the row.
__global__ __launch_bounds__(256) void combine_kernel(const f16 *__restrict__ y_perm,
                                                      const f16 *__restrict__ ys,
                                                      const int32_t *__restrict__ inv_pos,
                                                      const float *__restrict__ w, int k, int H,
                                                      int N, int rmsnorm, int renorm, float eps,
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
  if (renorm) renorm_weights(s_w, k);

  auto row_chunk = [&](int c, float (&v)[8]) {
    if (ys) {
      const f16x8 a = as_f16x8(ld16(ys + (size_t)t * H + c));
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    accumulate_rows(v, y_perm, H, c, k, [&](int j) { return s_row[j]; },
                    [&](int j) { return s_w[j]; });
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

// Without the norm the columns are independent: one 64-thread block per
// (token, 512 columns), so a small batch spreads over many CUs.
__global__ __launch_bounds__(64) void combine_cols_kernel(const f16 *__restrict__ y_perm,
                                                          const f16 *__restrict__ ys,
                                                          const int32_t *__restrict__ inv_pos,
                                                          const float *__restrict__ w, int k,
                                                          int H, int N, int renorm,
                                                          f16 *__restrict__ out) {
  const int chunks = (H + 511) / 512;
  const int t = blockIdx.x / chunks;
  const int c = (blockIdx.x % chunks) * 512 + threadIdx.x * 8;
  if (c >= H) return;
  // the shared expert's piece through a buffer over this token's row (empty
  // without a shared expert), so it loads (as zeros) with the row indices
  // and no branch; the row base is a 64-bit address, the offset within the
  // row at most 2 * 65536 bytes
  const rsrc_t yrs = make_rsrc(ys ? ys + (size_t)t * H : ys, ys ? (uint32_t)H * 2u : 0u);
  const u32x4 yraw = bload16(yrs, (uint32_t)c * 2u, 0);
  float wsum = 1.0f;
  if (renorm) {
    wsum = 0.0f;
    for (int j = 0; j < k; ++j) wsum += w[(size_t)t * k + j];
  }
  float v[8];
  accumulate_rows(
      v, y_perm, H, c, k,
      [&](int j) {
        const int r = inv_pos[(size_t)t * k + j];
        return r < 0 ? 0 : (r >= N ? N - 1 : r);
      },
      [&](int j) { return renorm ? w[(size_t)t * k + j] / wsum : w[(size_t)t * k + j]; },
      [&](float (&a)[8]) {
        const f16x8 h = as_f16x8(yraw);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = (float)h[i];
      });
  f16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (f16)v[i];
  *reinterpret_cast<f16x8 *>(out + (size_t)t * H + c) = o;
}

// With the norm, rows of up to 8192 columns: one block per token, one thread
// per 8 columns, the combined row kept in registers (formed once).
__global__ __launch_bounds__(1024) void combine_norm_kernel(const f16 *__restrict__ y_perm,
                                                            const f16 *__restrict__ ys,
                                                            const int32_t *__restrict__ inv_pos,
                                                            const float *__restrict__ w, int k,
                                                            int H, int N, int renorm, float eps,
                                                            f16 *__restrict__ out) {
  __shared__ int s_row[kMaxK];
  __shared__ float s_w[kMaxK];
  __shared__ float s_red[16];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid < k) {
    int r = inv_pos[(size_t)t * k + tid];
    s_row[tid] = r < 0 ? 0 : (r >= N ? N - 1 : r);
    s_w[tid] = w[(size_t)t * k + tid];
  }
  const int c = tid * 8;
  const bool live = c < H;
  float v[8];
  if (ys && live) {
    const f16x8 a = as_f16x8(ld16(ys + (size_t)t * H + c));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  __syncthreads();
  if (renorm) renorm_weights(s_w, k);
  if (live)
    accumulate_rows(v, y_perm, H, c, k, [&](int j) { return s_row[j]; },
                    [&](int j) { return s_w[j]; });
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  ss = wave_sum(ss);
  const int nw = blockDim.x / kWave;
  if ((tid & (kWave - 1)) == 0) s_red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int i = 0; i < nw; ++i) tot += s_red[i];        // fixed order
  const float scale = 1.0f / sqrtf(tot / (float)H + eps);
  if (live) {
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
  const int renorm = (flags & MOE_RENORM) ? 1 : 0;
  if (!(flags & MOE_RMSNORM)) {
    hipLaunchKernelGGL(combine_cols_kernel, dim3(T * ((H + 511) / 512)), dim3(64), 0, st,
                       reinterpret_cast<const f16 *>(y_perm),
                       reinterpret_cast<const f16 *>(y_shared), inv_pos, w, k, H, T * k,
                       renorm, reinterpret_cast<f16 *>(out));
    return hipGetLastError();
  }
  if (H <= 8192) {
    const int threads = ((H / 8 + kWave - 1) / kWave) * kWave;
    hipLaunchKernelGGL(combine_norm_kernel, dim3(T), dim3(threads), 0, st,
                       reinterpret_cast<const f16 *>(y_perm),
                       reinterpret_cast<const f16 *>(y_shared), inv_pos, w, k, H, T * k, renorm,
                       eps, reinterpret_cast<f16 *>(out));
    return hipGetLastError();
  }
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, st,
                     reinterpret_cast<const f16 *>(y_perm), reinterpret_cast<const f16 *>(y_shared),
                     inv_pos, w, k, H, T * k, (flags & MOE_RMSNORM) ? 1 : 0, renorm, eps,
                     reinterpret_cast<f16 *>(out));
  return hipGetLastError();
}

}  // namespace moe
