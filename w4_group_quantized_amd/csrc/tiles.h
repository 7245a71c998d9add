// Wave-level 16x16 MFMA tiles over a K range, for weights streamed from HBM.
//
// Operand roles (v_mfma_f32_16x16x32_f16): A = activations, 16 token rows;
// B = weights transposed, 16 weight rows as columns.  Lane l owns token row
// (l % 16) of A and weight row (l % 16) of B, and k-block kb = l / 16.  Within
// one 128-wide quantization group the lane covers the 32 consecutive columns
// [32*kb, 32*kb + 32) as four MFMAs of 8 columns each, so its int4 weights are
// one 16-byte load and its activations four 16-byte loads.  The accumulator
// lane l receives D[4*kb + j][l % 16], j = 0..3: tokens 4*kb + j of weight row
// l % 16, so each lane applies a single group scale per tile.
#pragma once

#include "common.h"

namespace moe {

// int4 weights: acc[t] += sum_g scale[t][g] * sum_{k in g} A[tok][k] * q[t][k]
// for g in [g0, g1).  arow: this lane's activation row (nullptr -> zeros);
// qrow[t]: this lane's packed weight row of tile t; srow[t]: its scales.
template <int NT>
__device__ __forceinline__ void w4_tiles(const f16 *__restrict__ arow,
                                         const uint8_t *const (&qrow)[NT],
                                         const f16 *const (&srow)[NT], int kb, int g0, int g1,
                                         f32x4 (&acc)[NT]) {
  if (g0 >= g1) return;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 xa[4], wq[NT];
  f16 sc[NT];
  auto load = [&](int g, u32x4 (&x)[4], u32x4 (&q)[NT], f16 (&s)[NT]) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      x[m] = arow ? ld16(arow + (size_t)g * kGroup + kb * 32 + m * 8) : zero;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      q[t] = ld16(qrow[t] + (size_t)g * (kGroup / 2) + kb * 16);
      s[t] = srow[t][g];
    }
  };
  load(g0, xa, wq, sc);
  for (int g = g0; g < g1; ++g) {
    u32x4 xn[4], qn[NT];
    f16 sn[NT];
    load(g + 1 < g1 ? g + 1 : g, xn, qn, sn);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) tmp = mfma_16x16x32(as_f16x8(xa[m]), unpack8(wq[t][m]), tmp);
      const float s = (float)sc[t];
      acc[t] += s * tmp;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) xa[m] = xn[m];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      wq[t] = qn[t];
      sc[t] = sn[t];
    }
  }
}

// fp16 weights: acc[t] += sum_{k in groups [g0, g1)} A[tok][k] * W[t][k].
template <int NT>
__device__ __forceinline__ void f16_tiles(const f16 *__restrict__ arow,
                                          const f16 *const (&wrow)[NT], int kb, int g0, int g1,
                                          f32x4 (&acc)[NT]) {
  if (g0 >= g1) return;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 xa[4], wb[NT][4];
  auto load = [&](int g, u32x4 (&x)[4], u32x4 (&w)[NT][4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const size_t k = (size_t)g * kGroup + kb * 32 + m * 8;
      x[m] = arow ? ld16(arow + k) : zero;
#pragma unroll
      for (int t = 0; t < NT; ++t) w[t][m] = ld16(wrow[t] + k);
    }
  };
  load(g0, xa, wb);
  for (int g = g0; g < g1; ++g) {
    u32x4 xn[4], wn[NT][4];
    load(g + 1 < g1 ? g + 1 : g, xn, wn);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[t] = mfma_16x16x32(as_f16x8(xa[m]), as_f16x8(wb[t][m]), acc[t]);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      xa[m] = xn[m];
#pragma unroll
      for (int t = 0; t < NT; ++t) wb[t][m] = wn[t][m];
    }
  }
}

// Sum the accumulators of the 4 waves of a block (K split 4 ways) into wave 0,
// in the fixed order wave 0 + 1 + 2 + 3.  red: LDS of 3 * NT * 4 * 64 floats.
template <int NT>
__device__ __forceinline__ void ksplit_reduce(f32x4 (&acc)[NT], float *red) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  if (wid > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[(((wid - 1) * NT + t) * 4 + j) * kWave + lane] = acc[t][j];
  }
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int w = 1; w < 4; ++w)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] += red[(((w - 1) * NT + t) * 4 + j) * kWave + lane];
  }
}

}  // namespace moe
