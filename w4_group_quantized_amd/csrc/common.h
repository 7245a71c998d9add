// Device helpers shared by the gfx950 kernels of the W4 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace moe {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kGroup = 128;   // weights per quantization group along in_features

// D[16x16] += A[16x32] * B[32x16], fp16 inputs, fp32 accumulation.
// Lane l supplies A row (l % 16) and B column (l % 16), 8 consecutive k each,
// k-block (l / 16); it receives D rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Register-resident constants for the unpack.  GFX9 VOP3 encodings take no
// literal constants, so with literal masks the compiler emits AND + OR; with
// the masks in SGPRs and the fp16 1024.0 pair in a VGPR (made opaque by an
// empty asm so they are not folded back into literals) it selects one
// v_and_or_b32 per pair.
struct UnpackConsts {
  uint32_t lo, hi, magic;
};
__device__ __forceinline__ UnpackConsts unpack_consts() {
  UnpackConsts c{0x000F000Fu, 0x00F000F0u, 0x64006400u};
  asm volatile("" : "+s"(c.lo), "+s"(c.hi));
  asm volatile("" : "+v"(c.magic));
  return c;
}

// Eight int4 codes of one 32-bit word of the packed format -> eight fp16
// codes q = u - 8 in column order.  Nibble p of the word holds column
// {0,2,4,6,1,3,5,7}[p], so masking bits 0-3 and 16-19 yields columns (0,1),
// bits 4-7 and 20-23 yields columns (2,3), and the same on the word shifted
// by 8 yields (4,5) and (6,7).  OR-ing a nibble into the mantissa of fp16
// 1024.0 (0x6400) gives 1024 + u exactly (fp16 spacing is 1 on [1024, 2048));
// a nibble sitting 4 bits higher gives 1024 + 16u.  One subtraction, or one
// fused multiply-add by 1/16, then leaves the exact small integer u - 8.
// Cost: 1 shift + 4 AND-OR + 4 packed fp16 ops per 8 weights.
__device__ __forceinline__ f16x8 unpack8(uint32_t w, const UnpackConsts &k) {
  const f16x2 k1032 = {(f16)-1032.0f, (f16)-1032.0f};
  const f16x2 k16th = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 k72 = {(f16)-72.0f, (f16)-72.0f};
  const uint32_t w8 = w >> 8;
  f16x2 c01 = as_f16x2((w & k.lo) | k.magic) + k1032;
  f16x2 c23 = __builtin_elementwise_fma(as_f16x2((w & k.hi) | k.magic), k16th, k72);
  f16x2 c45 = as_f16x2((w8 & k.lo) | k.magic) + k1032;
  f16x2 c67 = __builtin_elementwise_fma(as_f16x2((w8 & k.hi) | k.magic), k16th, k72);
  u32x4 r = {as_u32(c01), as_u32(c23), as_u32(c45), as_u32(c67)};
  return as_f16x8(r);
}

__device__ __forceinline__ u32x4 ldg16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over a block of `nthreads` threads (multiple of 64,
// at most 1024).  `scratch` holds at least nthreads/64 ints of LDS.  Returns
// this thread's exclusive prefix; *total receives the block sum.
__device__ __forceinline__ int block_excl_scan(int v, int *scratch, int *total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int incl = wave_incl_scan(v);
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    int s = scratch[i];
    if (i < wid) wbase += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

}  // namespace moe
