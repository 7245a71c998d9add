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
//
// The K loop is software-pipelined by hand: two register stages (ping-pong)
// of S quantization groups each; the loads of one stage are in flight while
// the other is unpacked and multiplied.  Scheduling barriers keep the
// compiler from sinking the prefetch loads next to their uses.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// The A operand rows of one tile: lane (r, kb) reads the 32 consecutive
// columns [32*kb, 32*kb + 32) of each 128-wide group of its token row through
// a raw buffer.  Lanes whose row is past the tile hold an offset beyond the
// buffer, so their loads return zeros without a memory access (their output
// rows are discarded).
struct ARows {
  rsrc_t rs;
  uint32_t voff;   // row byte offset + 64 * kb, or kPadOffset
  static constexpr uint32_t kPadOffset = 0x80000000u;
  // rows [0, nrows) of a [*, K] fp16 matrix at `base`, this lane's row `row`
  // (nrows * K * 2 < 2^31)
  __device__ __forceinline__ ARows(const f16 *base, int nrows, int K, int row, bool live, int kb)
      : rs(make_rsrc(base, (uint32_t)nrows * (uint32_t)K * 2u)),
        voff(live ? (uint32_t)row * (uint32_t)K * 2u + 64u * kb : kPadOffset) {}
  static constexpr bool kDeferred = false;   // loaded with the weights of its stage
  // 8 halfs at column 128*g + 32*kb + 8*m
  __device__ __forceinline__ u32x4 load(int g, int m) const {
    return bload16(rs, voff + 16u * m, (uint32_t)g * 256u);
  }
};

// The same A operand rows staged in LDS by the block (row stride `stride`
// bytes): read right before the MFMAs that use them.  Lanes past the tile
// read the last live row (their output rows are discarded).
template <int LDS_VEC>
struct ALds {
  const u32x4 (&lds)[LDS_VEC];
  uint32_t idx;    // this lane's row start + 64 * kb, in 16-byte units
  static constexpr bool kDeferred = true;
  __device__ __forceinline__ ALds(const u32x4 (&l)[LDS_VEC], int row, int stride, int kb)
      : lds(l), idx((uint32_t)(row * stride + 64 * kb) / 16u) {}
  __device__ __forceinline__ u32x4 load(int g, int m) const { return lds[idx + 16 * g + m]; }
};

// Quantization group size of the int4 weights.  The K loop always walks
// 128-column blocks (one 1 KB chunk per 16-row tile); the scale of a block
// is applied after its MFMAs when the block lies inside one group (128 and
// 256), and folded into the unpacked weights, RN16(q * s), when each lane's
// 32 columns have their own group (64: lanes kb = 0, 1 and kb = 2, 3 of a
// block read two different scales).
enum GroupMode { kG128 = 0, kG64 = 1, kG256 = 2 };

// Scale group of 128-column block gg (the lane's kb offset for kG64 is part
// of the caller's scale pointer).
template <int GM>
__device__ __forceinline__ int scale_group(int gg) {
  return GM == kG64 ? 2 * gg : (GM == kG256 ? gg >> 1 : gg);
}

// One pipeline stage of the int4 path: S groups of activations, weights and
// scales for NT weight tiles.
template <int NT, int S>
struct W4Stage {
  u32x4 x[S][4];
  u32x4 q[S][NT];
  f16 s[S][NT];
};

// Code loads: streamed (non-temporal) when no other tile of the launch reads
// the same weight lines, cached when segments span several 16-row tiles that
// each read the expert's weights (STREAM, chosen by the host).
template <bool STREAM>
__device__ __forceinline__ u32x4 ld16_codes(const void *p) {
  return STREAM ? ld16_stream(p) : ld16(p);
}

template <int NT, int S, int GM, bool STREAM, class A>
__device__ __forceinline__ void w4_load(W4Stage<NT, S> &st, const A &a,
                                        const uint8_t *const (&qrow)[NT],
                                        const f16 *const (&srow)[NT], int g, int G) {
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int gg = min(g + i, G - 1);   // past the end: reload the last group (never used)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      st.q[i][t] = ld16_codes<STREAM>(qrow[t] + (size_t)gg * 1024);   // 1 KB: 8 whole lines
      st.s[i][t] = srow[t][(size_t)scale_group<GM>(gg) * 16];
    }
    if (!A::kDeferred) {
#pragma unroll
      for (int m = 0; m < 4; ++m) st.x[i][m] = a.load(gg, m);
    }
  }
}

template <int NT, int S, int GM, class A>
__device__ __forceinline__ void w4_compute(const W4Stage<NT, S> &st, const A &a, int g, int ngroups,
                                           const UnpackConsts &magic, f32x4 (&acc)[NT]) {
#pragma unroll
  for (int i = 0; i < S; ++i) {
    if (i < ngroups) {
      u32x4 x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = A::kDeferred ? a.load(g + i, m) : st.x[i][m];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (GM == kG64) {       // RN16(q * s), accumulated straight into acc
          const f16 s = st.s[i][t];
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[t] = mfma_16x16x32(as_f16x8(x[m]), unpack8(st.q[i][t][m], magic) * s, acc[t]);
        } else {
          f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int m = 0; m < 4; ++m)
            tmp = mfma_16x16x32(as_f16x8(x[m]), unpack8(st.q[i][t][m], magic), tmp);
          const float s = (float)st.s[i][t];
          acc[t] += s * tmp;
        }
      }
    }
  }
}

// int4 weights: acc[t] += sum_g scale[t][g] * sum_{k in g} A[tok][k] * q[t][k]
// for 128-column blocks g in [g0, g1).  arow: this lane's activation rows
// (ARows or ALds); qrow[t]: base of weight tile t (16 rows) + lane*16 bytes,
// so block g is at qrow[t] + g*1024; srow[t]: the tile's scales + r (+ 16 for
// lanes kb = 2, 3 with 64-column groups), scale group sg at srow[t][sg*16].
// after_first() runs once the first stage's loads are issued (the block can
// stage its activations there while they are in flight).  The loop body has
// no control flow, so the two stages stay in fixed registers and only the
// stage about to be used is waited for.
struct NoOp {
  __device__ __forceinline__ void operator()() const {}
};
template <int NT, int S, int GM, bool STREAM, class A, class F = NoOp>
__device__ __forceinline__ void w4_tiles(const A &arow, const uint8_t *const (&qrow)[NT],
                                         const f16 *const (&srow)[NT], int g0, int g1,
                                         f32x4 (&acc)[NT], F after_first = F()) {
  if (g0 >= g1) return;
  const UnpackConsts magic = unpack_consts();
  W4Stage<NT, S> a, b;
  w4_load<NT, S, GM, STREAM>(a, arow, qrow, srow, g0, g1);
  after_first();
  int g = g0;
  for (; g + 2 * S <= g1; g += 2 * S) {
    w4_load<NT, S, GM, STREAM>(b, arow, qrow, srow, g + S, g1);
    sched_fence();
    w4_compute<NT, S, GM>(a, arow, g, S, magic, acc);
    sched_fence();
    w4_load<NT, S, GM, STREAM>(a, arow, qrow, srow, g + 2 * S, g1);
    sched_fence();
    w4_compute<NT, S, GM>(b, arow, g + S, S, magic, acc);
    sched_fence();
  }
  const int rest = g1 - g;          // 0 <= rest < 2S groups; stage a holds group g..
  if (rest > 0) {
    w4_compute<NT, S, GM>(a, arow, g, rest, magic, acc);
    if (rest > S) {
      w4_load<NT, S, GM, STREAM>(b, arow, qrow, srow, g + S, g1);
      w4_compute<NT, S, GM>(b, arow, g + S, rest - S, magic, acc);
    }
  }
}

// fp16 weights: acc[t] += sum_{k in groups [g0, g1)} A[tok][k] * W[t][k].
template <int NT>
struct F16Stage {
  u32x4 x[4];
  u32x4 w[NT][4];
};

template <int NT>
__device__ __forceinline__ void f16_load(F16Stage<NT> &st, const ARows &arow,
                                         const f16 *const (&wrow)[NT], int kb, int g, int G) {
  const int gg = min(g, G - 1);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const size_t k = (size_t)gg * kGroup + kb * 32 + m * 8;
    st.x[m] = arow.load(gg, m);
#pragma unroll
    for (int t = 0; t < NT; ++t) st.w[t][m] = ld16(wrow[t] + k);
  }
}

template <int NT>
__device__ __forceinline__ void f16_compute(const F16Stage<NT> &st, f32x4 (&acc)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[t] = mfma_16x16x32(as_f16x8(st.x[m]), as_f16x8(st.w[t][m]), acc[t]);
}

template <int NT>
__device__ __forceinline__ void f16_tiles(const ARows &arow,
                                          const f16 *const (&wrow)[NT], int kb, int g0, int g1,
                                          f32x4 (&acc)[NT]) {
  if (g0 >= g1) return;
  F16Stage<NT> a, b;
  f16_load<NT>(a, arow, wrow, kb, g0, g1);
  int g = g0;
  for (; g + 2 <= g1; g += 2) {
    f16_load<NT>(b, arow, wrow, kb, g + 1, g1);
    sched_fence();
    f16_compute<NT>(a, acc);
    sched_fence();
    f16_load<NT>(a, arow, wrow, kb, g + 2, g1);
    sched_fence();
    f16_compute<NT>(b, acc);
    sched_fence();
  }
  if (g < g1) f16_compute<NT>(a, acc);
}

// 8-bit weights (the shared expert's W8 g128 format: offset-binary bytes,
// 16-row tiles of 16-column chunks, 2 KB per tile and 128-column block).
// Lane (r, kb) holds the 32 bytes of columns [32kb, 32kb + 32) of weight row
// r in a block: chunks 2kb and 2kb+1, 256 bytes apart; MFMA m uses bytes
// 8m .. 8m+7, the same columns as the activation piece m.  The codes become
// exact fp16 values: byte b is placed under the exponent byte 0x64 (giving
// 1024 + b) and 1152 is subtracted.  One fp16 scale per row and block,
// applied to the block's product in fp32.
__device__ __forceinline__ f16x8 unpack_i8x8(uint32_t lo, uint32_t hi) {
  constexpr uint32_t kHi = 0x64646464u;
  u32x4 v;
  // byte selectors: 0..3 pick bytes of the second operand, 4..7 of the first
  v[0] = __builtin_amdgcn_perm(kHi, lo, 0x05010400u);
  v[1] = __builtin_amdgcn_perm(kHi, lo, 0x05030402u);
  v[2] = __builtin_amdgcn_perm(kHi, hi, 0x05010400u);
  v[3] = __builtin_amdgcn_perm(kHi, hi, 0x05030402u);
  return as_f16x8(v) - (f16)1152.0f;
}

template <int NT>
struct W8Stage {
  u32x4 x[4];
  u32x4 q[NT][2];
  f16 s[NT];
};

template <int NT, bool STREAM>
__device__ __forceinline__ void w8_load(W8Stage<NT> &st, const ARows &arow,
                                        const uint8_t *const (&qrow)[NT],
                                        const f16 *const (&srow)[NT], int g, int G) {
  const int gg = min(g, G - 1);   // past the end: reload the last block (never used)
#pragma unroll
  for (int m = 0; m < 4; ++m) st.x[m] = arow.load(gg, m);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st.q[t][0] = ld16_codes<STREAM>(qrow[t] + (size_t)gg * 2048);   // whole lines each
    st.q[t][1] = ld16_codes<STREAM>(qrow[t] + (size_t)gg * 2048 + 256);
    st.s[t] = srow[t][(size_t)gg * 16];
  }
}

template <int NT>
__device__ __forceinline__ void w8_compute(const W8Stage<NT> &st, f32x4 (&acc)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const u32x4 &c = st.q[t][m >> 1];
      tmp = mfma_16x16x32(as_f16x8(st.x[m]), unpack_i8x8(c[2 * (m & 1)], c[2 * (m & 1) + 1]), tmp);
    }
    acc[t] += (float)st.s[t] * tmp;
  }
}

// 8-bit weights: acc[t] += sum_g scale[t][g] * sum_{k in g} A[tok][k] * q[t][k]
// over blocks [g0, g1); qrow[t]: tile base + 2kb*256 + r*16 (block g at
// + g*2048); srow[t]: the tile's scales + r (block g at srow[t][g*16]).
template <int NT, bool STREAM>
__device__ __forceinline__ void w8_tiles(const ARows &arow, const uint8_t *const (&qrow)[NT],
                                         const f16 *const (&srow)[NT], int g0, int g1,
                                         f32x4 (&acc)[NT]) {
  if (g0 >= g1) return;
  W8Stage<NT> a, b;
  w8_load<NT, STREAM>(a, arow, qrow, srow, g0, g1);
  int g = g0;
  for (; g + 2 <= g1; g += 2) {
    w8_load<NT, STREAM>(b, arow, qrow, srow, g + 1, g1);
    sched_fence();
    w8_compute<NT>(a, acc);
    sched_fence();
    w8_load<NT, STREAM>(a, arow, qrow, srow, g + 2, g1);
    sched_fence();
    w8_compute<NT>(b, acc);
    sched_fence();
  }
  if (g < g1) w8_compute<NT>(a, acc);
}

// Sum the accumulators of the NW waves of a block (K split NW ways) into wave
// 0, in the fixed order wave 0 + 1 + ... + NW-1.
// red: LDS of (NW - 1) * NT * 4 * 64 floats.
template <int NT, int NW = 4>
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
    for (int w = 1; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] += red[(((w - 1) * NT + t) * 4 + j) * kWave + lane];
  }
}

}  // namespace moe
