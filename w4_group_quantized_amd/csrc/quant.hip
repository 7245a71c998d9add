// Group quantization (fp16 -> packed int4 + fp16 scales) and the exact
// dequantization test hook.
//
// Quantizer: lpnh.cn/news/2730718 §2.1 (group-quantization pseudo-code),
// applied to fp16 weights (§3.2), so each arithmetic step rounds to fp16:
//   s = RN16(max|w| / 7),  q = clamp(RNE(RN16(w / s)), -8, 7);  s = 0 -> q = 0.
// Quotients are formed with the correctly rounded fp32 division and then
// rounded to fp16; with 24 >= 2*11 + 2 bits that double rounding equals a
// single correct rounding to fp16.
#include "common.h"
#include "kernels.h"

namespace moe {

// Stored layout (see the packed-weight format in moe_w4.h): 16 rows side by
// side per 16-byte chunk of 32 columns, so one group of a 16-row tile is 1 KB
// contiguous; scales likewise 16 rows side by side per group.
__device__ __forceinline__ size_t word_offset(int64_t row, int64_t word, int64_t cols) {
  // word = 8-column word index within the row; 4 words per 16-byte chunk
  return (size_t)(row >> 4) * 16 * (cols / 2) + (size_t)(word >> 2) * 256 +
         (size_t)(row & 15) * 16 + (size_t)(word & 3) * 4;
}
__device__ __forceinline__ size_t scale_offset(int64_t row, int64_t g, int64_t cols, int gs) {
  return (size_t)(row >> 4) * 16 * (cols / gs) + (size_t)g * 16 + (size_t)(row & 15);
}

// One thread per 8 consecutive columns (one 32-bit packed word); gs/8
// consecutive lanes (8, 16 or 32) cover one group of gs columns.  A row holds
// a whole number of groups, so no group straddles two waves.
__global__ __launch_bounds__(256) void quantize_kernel(const f16 *__restrict__ w,
                                                       int64_t rows, int64_t cols, int gs,
                                                       uint8_t *__restrict__ q,
                                                       f16 *__restrict__ s) {
  const int64_t words_per_row = cols / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = rows * words_per_row;
  // Lanes past the end still take part in the group max so that the
  // shuffles see a full group; they load nothing and store nothing.
  const bool live = t < total;
  const int64_t row = live ? t / words_per_row : 0, word = live ? t % words_per_row : 0;
  float v[8];
  float m = 0.0f;
  if (live) {
    u32x4 raw = ld16(w + row * cols + word * 8);
    f16x8 h = as_f16x8(raw);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = (float)h[i];
      m = fmaxf(m, fabsf(v[i]));
    }
  }
  const int glanes = gs / 8;
  for (int o = 1; o < glanes; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  if (!live) return;
  const f16 s16 = (f16)__fdiv_rn(m, 7.0f);
  const float sf = (float)s16;
  uint32_t u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float qi = 0.0f;
    if (sf > 0.0f) {
      const f16 r16 = (f16)__fdiv_rn(v[i], sf);
      qi = fminf(fmaxf(rintf((float)r16), -8.0f), 7.0f);
    }
    u[i] = (uint32_t)((int)qi + 8);
  }
  // nibble p holds column {0,2,4,6,1,3,5,7}[p]
  const uint32_t packed = u[0] | (u[2] << 4) | (u[4] << 8) | (u[6] << 12) | (u[1] << 16) |
                          (u[3] << 20) | (u[5] << 24) | (u[7] << 28);
  *reinterpret_cast<uint32_t *>(q + word_offset(row, word, cols)) = packed;
  if (word % glanes == 0) s[scale_offset(row, word / glanes, cols, gs)] = s16;
}

// Codes already quantized, in the plain row-major layout (byte c/2 of a row
// holds column c in bits 0-3 and column c+1 in bits 4-7, two's-complement
// nibbles; scales row-major [rows, cols/gs]) -> the stored format.  One thread
// per 8 columns: the input word's low nibbles are columns 0,2,4,6 and its high
// nibbles 1,3,5,7, which is the stored word's nibble order once each half is
// compacted; XOR 0x8 per nibble turns two's complement into offset binary.
__global__ __launch_bounds__(256) void pack_kernel(const uint32_t *__restrict__ q_rm,
                                                   const f16 *__restrict__ s_rm,
                                                   int64_t rows, int64_t cols, int gs,
                                                   uint8_t *__restrict__ q,
                                                   f16 *__restrict__ s) {
  const int64_t words_per_row = cols / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * words_per_row) return;
  const int64_t row = t / words_per_row, word = t % words_per_row;
  const uint32_t in = q_rm[t];                  // row-major: word t is row `row`, word `word`
  uint32_t lo = in & 0x0F0F0F0Fu;               // columns 0,2,4,6 in the low nibble of each byte
  uint32_t hi = (in >> 4) & 0x0F0F0F0Fu;        // columns 1,3,5,7
  lo = (lo | (lo >> 4)) & 0x00FF00FFu;
  lo = (lo | (lo >> 8)) & 0x0000FFFFu;
  hi = (hi | (hi >> 4)) & 0x00FF00FFu;
  hi = (hi | (hi >> 8)) & 0x0000FFFFu;
  *reinterpret_cast<uint32_t *>(q + word_offset(row, word, cols)) = (lo | (hi << 16)) ^ 0x88888888u;
  const int glanes = gs / 8;
  if (word % glanes == 0)
    s[scale_offset(row, word / glanes, cols, gs)] = s_rm[row * (cols / gs) + word / glanes];
}

// out[n][c] = q[n][c] * s[n][c/gs] in fp32 (exact), decoding with the same
// unpack8() the FFN kernels use.  One thread per stored 32-bit word.
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *__restrict__ q,
                                                      const f16 *__restrict__ s,
                                                      int64_t rows, int64_t cols, int gs,
                                                      float *__restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * (cols / 8)) return;
  const int64_t byte = t * 4;
  const int64_t tile_bytes = 16 * (cols / 2);
  const int64_t tile = byte / tile_bytes, rem = byte % tile_bytes;
  const int64_t chunk = rem / 256, r = (rem % 256) / 16, word_in_chunk = (rem % 16) / 4;
  const int64_t row = tile * 16 + r;
  const int64_t col = chunk * 32 + word_in_chunk * 8;
  const float sc = (float)s[scale_offset(row, col / gs, cols, gs)];
  const f16x8 c = unpack8(q[t], unpack_consts());
  f32x4 a = {(float)c[0] * sc, (float)c[1] * sc, (float)c[2] * sc, (float)c[3] * sc};
  f32x4 b = {(float)c[4] * sc, (float)c[5] * sc, (float)c[6] * sc, (float)c[7] * sc};
  f32x4 *o = reinterpret_cast<f32x4 *>(out + row * cols + col);
  o[0] = a;
  o[1] = b;
}

// 8-bit codes for the shared expert (xdnf.cn/news/329730 §3.1: shared FFN at
// 8 bits, 128-weight groups): the same steps with 127 and [-128, 127]; the
// byte q + 128 of column c of row n goes to (n/16)*16*cols + (c/16)*256 +
// (n%16)*16 + c%16, so a thread's 8 columns are one aligned 8-byte store.
__global__ __launch_bounds__(256) void quantize8_kernel(const f16 *__restrict__ w,
                                                        int64_t rows, int64_t cols,
                                                        uint8_t *__restrict__ q,
                                                        f16 *__restrict__ s) {
  const int64_t words_per_row = cols / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = t < rows * words_per_row;
  const int64_t row = live ? t / words_per_row : 0, word = live ? t % words_per_row : 0;
  float v[8];
  float m = 0.0f;
  if (live) {
    const f16x8 h = as_f16x8(ld16(w + row * cols + word * 8));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = (float)h[i];
      m = fmaxf(m, fabsf(v[i]));
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));   // 16 lanes = 128 columns
  if (!live) return;
  const f16 s16 = (f16)__fdiv_rn(m, 127.0f);
  const float sf = (float)s16;
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float qi = 0.0f;
    if (sf > 0.0f) {
      const f16 r16 = (f16)__fdiv_rn(v[i], sf);
      qi = fminf(fmaxf(rintf((float)r16), -128.0f), 127.0f);
    }
    b[i] = (uint32_t)((int)qi + 128);
  }
  uint2 packed;
  packed.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
  packed.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
  const int64_t col = word * 8;
  *reinterpret_cast<uint2 *>(q + (size_t)(row >> 4) * 16 * cols + (size_t)(col >> 4) * 256 +
                             (size_t)(row & 15) * 16 + (size_t)(col & 15)) = packed;
  if ((word & 15) == 0) s[scale_offset(row, word / 16, cols, 128)] = s16;
}

hipError_t launch_quantize8(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *q,
                            uint16_t *s, hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(quantize8_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const f16 *>(w), rows, cols, q, reinterpret_cast<f16 *>(s));
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t *w, int64_t rows, int64_t cols, int gs, uint8_t *q,
                           uint16_t *s, hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const f16 *>(w), rows, cols, gs, q,
                     reinterpret_cast<f16 *>(s));
  return hipGetLastError();
}

hipError_t launch_pack(const uint8_t *q_rm, const uint16_t *s_rm, int64_t rows, int64_t cols,
                       int gs, uint8_t *q, uint16_t *s, hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t *>(q_rm), reinterpret_cast<const f16 *>(s_rm),
                     rows, cols, gs, q, reinterpret_cast<f16 *>(s));
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *q, const uint16_t *s, int64_t rows, int64_t cols, int gs,
                          float *out, hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint32_t *>(q), reinterpret_cast<const f16 *>(s),
                     rows, cols, gs, out);
  return hipGetLastError();
}

}  // namespace moe
