// Shared by the decode FFN's kernels (ffn.hip: whole items; ffn_split.hip:
// items split in K over blocks): work-item arguments, tile constants and the
// per-block tile lookup.
#pragma once

#include "common.h"
#include "kernels.h"
#include "tiles.h"
#include "split_plan.h"

namespace moe {

constexpr int kTileM = 16;   // tokens per MFMA tile
// Token rows of a routed tile are staged in LDS when they take at most this
// many bytes (each of the 256 threads moves kStagePieces 16-byte pieces).
constexpr int kStagePieces = 8;
constexpr int kActLdsBytes = kStagePieces * 256 * 16;
constexpr int kActLdsVec = (kActLdsBytes + kTileM * 16) / 16;   // + row padding

struct FfnArgs {
  int E, H, F, Fs, T, N, k;         // N = T * k
  const int32_t *offsets;           // [E+1]
  const int32_t *perm_src;          // phase 1 without x_perm: rows of x via perm_src[r] / k
  const f16 *a_routed;              // phase 1: x_perm [N, H] or x [T, H]; phase 2: h [N, F]
  const f16 *a_shared;              // phase 1: x [T, H];      phase 2: h_shared [T, Fs]
  const uint8_t *q0, *q1;           // phase 1: gate_q, up_q;  phase 2: down_q, unused
  const f16 *s0, *s1;               // matching scales
  const f16 *w0, *w1;               // shared expert fp16 weights (phase 2: w0 only)
  const uint8_t *wq0, *wq1;         // or its 8-bit codes (shared_w8) ...
  const f16 *ws0, *ws1;             // ... and their g128 scales
  int shared_w8;
  f16 *out_routed;                  // phase 1: h [N, F];      phase 2: y_perm [N, H]
  f16 *out_shared;                  // phase 1: h_shared;      phase 2: y_shared
  int shared_items;                 // shared-expert items (their blocks first)
  int routed_items;                 // worst-case number of routed items (their blocks after)
  int rparts, sparts;               // blocks per routed / shared item (K parts; 1 = whole K)
  int tm;                           // token rows per tile kept in the partial sums
  float *part;                      // K-split partial sums: [block][wave][tile][tm][16]
  unsigned int *ticket;             // per item (shared items first): parts done, zero between calls
};

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Block-cooperative: which expert and which 16-row tile of its segment is
// segment tile `slot`?  Tiles are numbered expert by expert.  Returns false
// when slot is past the last tile.  Requires blockDim.x = 256, E <= 1024.
__device__ bool locate_tile(const int32_t *__restrict__ off, int E, int slot, int *e_out,
                            int *mt_out) {
  __shared__ int s_scan[4];
  __shared__ int s_res[2];
  const int tid = threadIdx.x;
  // five independent loads with clamped (in-bounds) indices, then the counts
  int o[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) o[i] = off[min(4 * tid + i, E)];
  int c[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    c[i] = e < E ? (o[i + 1] - o[i] + kTileM - 1) / kTileM : 0;
    sum += c[i];
  }
  int total;
  int run = block_excl_scan(sum, s_scan, &total);
  if (tid == 0) s_res[0] = -1;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (slot >= run && slot < run + c[i]) {
      s_res[0] = 4 * tid + i;
      s_res[1] = slot - run;
    }
    run += c[i];
  }
  __syncthreads();
  *e_out = s_res[0];
  *mt_out = s_res[1];
  return s_res[0] >= 0;
}

// Launch the K-split decode kernel of one phase (1: gate/up, 2: down) with NT
// 16-row tiles per wave (phase 1: 1 or 2; phase 2: 2 or 4) over `blocks`
// blocks.
hipError_t launch_ffn_split(int phase, int nt, int group_size, int blocks, const FfnArgs &a,
                            hipStream_t st);

}  // namespace moe
