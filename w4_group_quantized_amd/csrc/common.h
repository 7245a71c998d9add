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
constexpr int kGroup = 128;   // columns per K block: one 1 KB chunk of a 16-row int4 tile

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

// Raw buffer over `bytes` bytes at `base` (gfx9 descriptor: stride 0, plain
// dword data format).  Loads through it take a 32-bit per-lane byte offset
// plus a wave-uniform one in an SGPR; offsets past `bytes` read zeros and
// stores there are dropped.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// cache-policy operand of the buffer intrinsics: sc1, the device coherence
// point (what agent-scope atomic loads use on this target)
constexpr int kBufCoherent = 16;
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ f16 bload_f16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f16, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}

__device__ __forceinline__ u32x4 ldg16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
// All LDS operations of this wave are done; meet the other waves of the
// block.  Vector-memory loads stay in flight (no vmcnt wait, which
// __syncthreads would add); the "memory" clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
// A 16-byte load marked non-temporal (streamed: not kept in the caches).
// For weight bytes read exactly once, by one instruction per cache line:
// on the decode FFN it raised the HBM rate by 7-9% (the int4 codes); where
// two instructions read parts of one line (the fp16 shared-expert rows) it
// made the line come from memory twice.
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
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

// Routing key of one (logit, expert) candidate: the 64-bit maximum over a
// wave picks the largest logit, ties to the lower expert index, NaN below
// every number, and a key of 0 (empty or already chosen) below everything.
// High word: the float's bits mapped to an unsigned order (-0 folded into +0,
// NaN -> 0); low word: 1 << 16 | (0xFFFF - expert).
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  v = v + 0.0f;                                   // -0 -> +0
  uint32_t b = __float_as_uint(v);
  uint32_t m = (v != v) ? 0u : ((b >> 31) ? ~b : (b | 0x80000000u));
  return ((uint64_t)m << 32) | (1u << 16) | (uint32_t)(0xFFFF - e);
}
__device__ __forceinline__ int route_key_expert(uint64_t key) {
  return 0xFFFF - (int)(key & 0xFFFFu);
}
// The logit of a key: the inverse of the high word's order map (exact, but
// for -0, which comes back as +0, and NaN, which comes back as a NaN).
__device__ __forceinline__ float route_key_value(uint64_t key) {
  const uint32_t m = (uint32_t)(key >> 32);
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}
// Cross-lane reductions on DPP row operations (no LDS round trips): within
// each row of 16 lanes, exchange with lane^1, lane^2, the mirrored lane of the
// half row and of the row; afterwards every lane of a row holds the row's
// result.  The four row results are then combined on the scalar unit in row
// order, so every lane gets the same, order-fixed result.
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror
constexpr int kDppMirror = 0x140;       // row_mirror
constexpr int kDppRowBcast15 = 0x142;   // row_bcast:15 (lane 15 of the previous row)
constexpr int kDppRowBcast31 = 0x143;   // row_bcast:31 (lane 31, into rows 2 and 3)

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64_step(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)v), hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
  const uint64_t t = ((uint64_t)hi << 32) | lo;
  return t > v ? t : v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64_step<kDppXor1>(v);
  v = dpp_max_u64_step<kDppXor2>(v);
  v = dpp_max_u64_step<kDppHalfMirror>(v);
  v = dpp_max_u64_step<kDppMirror>(v);
  uint64_t r = 0;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, row * 16);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), row * 16);
    const uint64_t t = ((uint64_t)hi << 32) | lo;
    r = t > r ? t : r;
  }
  return r;
}

// Every lane holds its 16-lane row's maximum after the first four steps;
// row_bcast:15 then folds row 0 into row 1 and row 2 into row 3 (row mask
// 0b1010), row_bcast:31 folds lane 31 (rows 0-1) into rows 2 and 3 (row mask
// 0b1100), so lane 63 holds the wave's maximum: one read-lane instead of four.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppXor1>(v));
  v = max(v, dpp_u32<kDppXor2>(v));
  v = max(v, dpp_u32<kDppHalfMirror>(v));
  v = max(v, dpp_u32<kDppMirror>(v));
  // rows outside the row mask keep v (the "old" operand): max(v, v) = v
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowBcast15, 0xA, 0xF,
                                                   false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowBcast31, 0xC, 0xF,
                                                   false));
  return __builtin_amdgcn_readlane(v, 63);
}

// max that propagates NaN
__device__ __forceinline__ float fmax_nan(float a, float b) {
  return (a != a || b != b) ? __builtin_nanf("") : fmaxf(a, b);
}

__device__ __forceinline__ float wave_max_nan_dpp(float v) {
  v = fmax_nan(v, dpp_f32<kDppXor1>(v));
  v = fmax_nan(v, dpp_f32<kDppXor2>(v));
  v = fmax_nan(v, dpp_f32<kDppHalfMirror>(v));
  v = fmax_nan(v, dpp_f32<kDppMirror>(v));
  float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
#pragma unroll
  for (int row = 1; row < 4; ++row)
    r = fmax_nan(r, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), row * 16)));
  return r;
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = v + dpp_f32<kDppXor1>(v);
  v = v + dpp_f32<kDppXor2>(v);
  v = v + dpp_f32<kDppHalfMirror>(v);
  v = v + dpp_f32<kDppMirror>(v);
  float r = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
#pragma unroll
  for (int row = 1; row < 4; ++row)
    r = r + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), row * 16));
  return r;
}

}  // namespace moe
