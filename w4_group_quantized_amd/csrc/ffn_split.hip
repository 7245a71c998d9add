// The decode FFN with each work item's K range split over several blocks
// (small batches: see the host's rule with launch_ffn in ffn.hip).  Each
// block of an item computes the fp32 products of its share of the
// quantization groups; the item's last block adds the parts in a fixed order
// and applies the epilogue.  The arithmetic per group is the whole-item
// kernel's (ffn.hip).
//
// A translation unit of its own: with this kernel in the same module, the
// whole-item kernel's streamed instances were scheduled differently (more
// registers, address arithmetic inside the K loop) and ran 2% slower on the
// fine-grained layers, although their source was unchanged.
#include "ffn_decode.h"

namespace moe {

// K split over blocks: every block of an item stores the partial sums of the
// tile rows of its live tokens, and the last block of the item to take a
// ticket adds the parts in the fixed order 0 .. nparts-1 into acc.  The stores
// are agent-scope atomic stores (written through to the device coherence
// point); waiting for them before the barrier that precedes the ticket orders
// them before it, and the last block reads them with coherent (sc1) loads, as
// the one-launch router does with its logits.  Every wave of the block calls
// this; has_acc: this wave holds partial sums (with the K range split over the
// waves inside the block, only wave 0 after the in-block reduction).  Returns
// false in every block but the last, which also resets the ticket.
template <int NTL>
__device__ bool split_sum(f32x4 (&acc)[NTL], bool has_acc, int rows, int tm, float *item_part,
                          int blk_floats, int kpart, int nparts, unsigned int *ticket) {
  __shared__ int s_last;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int r = lane & 15, kb = lane >> 4;
  const int wave_floats = NTL * tm * 16;
  if (has_acc) {
    float *dst = item_part + (size_t)kpart * blk_floats + wid * wave_floats;
#pragma unroll
    for (int i = 0; i < NTL; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = 4 * kb + j;
        if (tok < rows)
          __hip_atomic_store(dst + (i * tm + tok) * 16 + r, acc[i][j], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(nparts - 1);
  __syncthreads();
  if (!s_last) return false;
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (has_acc) {
    const rsrc_t rs = make_rsrc(item_part, (uint32_t)(nparts * blk_floats) * 4u);
#pragma unroll
    for (int i = 0; i < NTL; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = 4 * kb + j;
        // parts past nparts and rows past the tile read zeros (out of range)
        float v[kMaxParts];
#pragma unroll
        for (int q = 0; q < kMaxParts; ++q) {
          const uint32_t off = tok < rows && q < nparts
                                   ? (uint32_t)(q * blk_floats + wid * wave_floats +
                                                (i * tm + tok) * 16 + r) * 4u
                                   : ARows::kPadOffset;
          v[q] = __builtin_bit_cast(float,
                                    __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kBufCoherent));
        }
        float sum = v[0];
#pragma unroll
        for (int q = 1; q < kMaxParts; ++q)
          if (q < nparts) sum += v[q];
        acc[i][j] = sum;
      }
  }
  return true;
}

// The whole-item kernel's work items (ffn.hip) with their K range split over
// p.rparts (routed) and p.sparts (shared) blocks, code loads streamed; item
// b's blocks are consecutive, shared items first.
template <int PHASE, int NT, int S, int GM>
__global__ __launch_bounds__(256) void ffn_split_kernel(FfnArgs p) {
  constexpr bool STREAM = true;
  constexpr bool kPair = PHASE == 1;
  constexpr int kMats = kPair ? 2 : 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int r = lane & 15, kb = lane >> 4;
  const int K = kPair ? p.H : p.F;             // in_features of this phase
  const int Nrows = kPair ? p.F : p.H;         // out_features of this phase
  const int G = K / kGroup;
  __shared__ float red[3 * 2 * 4 * kWave];
  __shared__ u32x4 s_act[kActLdsVec];

  const int rparts = p.rparts, sparts = p.sparts;
  const int sblocks = p.shared_items * sparts;
  // partial-sum floats per block (routed and shared blocks alike)
  const int blk_floats = 4 * kMats * NT * p.tm * 16;
  if ((int)blockIdx.x >= sblocks) {
    const int rb = blockIdx.x - sblocks;
    const int item = rb / rparts, kpart = rb - item * rparts;
    const int ntiles = Nrows / (64 * NT);
    const int slot = item / ntiles, nt = item % ntiles;
    int e, mt;
    if (!locate_tile(p.offsets, p.E, slot, &e, &mt)) return;
    const int seg0 = p.offsets[e] + mt * kTileM;
    // offsets come from device memory: keep every row inside [0, N)
    if (seg0 < 0 || seg0 >= p.N) return;
    const int rows = min(min(kTileM, p.offsets[e + 1] - seg0), p.N - seg0);
    const uint8_t *qrow[kMats * NT];
    const f16 *srow[kMats * NT];
    int nrow[NT];
    // scale groups per row, and this lane's scale within a 64-column pair
    const int Gs = GM == kG64 ? 2 * G : (GM == kG256 ? G / 2 : G);
    const int sl = r + (GM == kG64 ? (kb >> 1) * 16 : 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      nrow[t] = nt * 64 * NT + (wid * NT + t) * 16 + r;
      const size_t row0 = (size_t)e * Nrows + (nrow[t] - r);      // first row of the tile
      qrow[t] = p.q0 + row0 * (K / 2) + lane * 16;
      srow[t] = p.s0 + row0 * Gs + sl;
      if (kPair) {
        qrow[NT + t] = p.q1 + row0 * (K / 2) + lane * 16;
        srow[NT + t] = p.s1 + row0 * Gs + sl;
      }
    }
    f32x4 acc[kMats * NT];
#pragma unroll
    for (int t = 0; t < kMats * NT; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
    const int g0 = kpart * G / rparts, g1 = (kpart + 1) * G / rparts;
    const int KB = K * 2;                 // bytes per activation row
    if (rows * KB <= kActLdsBytes) {      // block-uniform
      // Stage the tile's token rows in LDS once for the four waves: the
      // loads go out before the first weight stage, the LDS writes after it,
      // so the weights are already in flight while the rows arrive.
      const int ppr = KB / 16;            // 16-byte pieces per row
      const int npieces = rows * ppr;
      const int stride = KB + 16;         // padded: rows start 4 banks apart
      const int tid = threadIdx.x;
      rsrc_t rs;
      uint32_t voff[kStagePieces];
      if (p.perm_src) {                   // gather straight from x
        rs = make_rsrc(p.a_routed, (uint32_t)p.T * (uint32_t)KB);
#pragma unroll
        for (int j = 0; j < kStagePieces; ++j) {
          const int i = j * 256 + tid;
          const int row = min(i / ppr, rows - 1);
          int tok = p.perm_src[seg0 + row] / p.k;
          tok = tok < 0 ? 0 : (tok >= p.T ? p.T - 1 : tok);
          voff[j] = i < npieces ? (uint32_t)tok * KB + (uint32_t)(i - row * ppr) * 16u
                                : ARows::kPadOffset;
        }
      } else {                            // rows seg0 .. seg0+rows-1 are contiguous
        rs = make_rsrc(p.a_routed + (size_t)seg0 * K, (uint32_t)rows * (uint32_t)KB);
#pragma unroll
        for (int j = 0; j < kStagePieces; ++j) {
          const int i = j * 256 + tid;
          voff[j] = i < npieces ? (uint32_t)i * 16u : ARows::kPadOffset;
        }
      }
      u32x4 stg[kStagePieces];
#pragma unroll
      for (int j = 0; j < kStagePieces; ++j) stg[j] = bload16(rs, voff[j], 0);
      const ALds<kActLdsVec> al(s_act, min(r, rows - 1), stride, kb);
      w4_tiles<kMats * NT, S, GM, STREAM>(al, qrow, srow, g0, g1, acc, [&] {
#pragma unroll
        for (int j = 0; j < kStagePieces; ++j) {
          const int i = j * 256 + tid;
          if (i < npieces) {
            const int row = i / ppr;
            s_act[(row * stride + (i - row * ppr) * 16) / 16] = stg[j];
          }
        }
        lds_barrier();
      });
    } else {
      // lanes of token rows past the tile read zeros; their outputs are dropped
      const bool live = r < rows;
      int tok = min(r, rows - 1);
      if (p.perm_src) {          // gather straight from x: token of flat index perm_src[r]
        tok = p.perm_src[seg0 + tok] / p.k;
        tok = tok < 0 ? 0 : (tok >= p.T ? p.T - 1 : tok);
      }
      const ARows arow = p.perm_src
                             ? ARows(p.a_routed, p.T, K, tok, live, kb)
                             : ARows(p.a_routed + (size_t)seg0 * K, rows, K, tok, live, kb);
      w4_tiles<kMats * NT, S, GM, STREAM>(arow, qrow, srow, g0, g1, acc);
    }
    if (rparts > 1 &&
        !split_sum<kMats * NT>(acc, true, rows, p.tm,
                               p.part + (size_t)(sblocks + item * rparts) * blk_floats,
                               blk_floats, kpart, rparts, p.ticket + p.shared_items + item))
      return;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = 4 * kb + j;
        if (tok < rows) {
          const float v = kPair ? silu(acc[t][j]) * acc[NT + t][j] : acc[t][j];
          p.out_routed[(size_t)(seg0 + tok) * Nrows + nrow[t]] = (f16)v;
        }
      }
    return;
  }

  // shared expert: fp16 weights (layers with the 8-bit shared expert are
  // never split), 16 weight rows per block, K split over waves
  const int Ks = kPair ? p.H : p.Fs;
  const int Ns = kPair ? p.Fs : p.H;
  const int Gs = Ks / kGroup;
  const int sitem = blockIdx.x / sparts, spart = blockIdx.x - sitem * sparts;
  const int sntiles = Ns / 16;
  const int mt = sitem / sntiles, nt = sitem % sntiles;
  const int tok0 = mt * kTileM;
  if (tok0 >= p.T) return;
  const int rows = min(kTileM, p.T - tok0);
  const ARows arow(p.a_shared + (size_t)tok0 * Ks, rows, Ks, r, r < rows, kb);
  const int nrow = nt * 16 + r;
  f32x4 acc[kMats];
#pragma unroll
  for (int t = 0; t < kMats; ++t) acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // this block's part of K, split again over its 4 waves
  const int lo = spart * Gs / sparts, hi = (spart + 1) * Gs / sparts;
  const int g0 = lo + wid * (hi - lo) / 4, g1 = lo + (wid + 1) * (hi - lo) / 4;
  {
    const f16 *wrow[kMats];
    wrow[0] = p.w0 + (size_t)nrow * Ks;
    if (kPair) wrow[kMats - 1] = p.w1 + (size_t)nrow * Ks;
    f16_tiles<kMats>(arow, wrow, kb, g0, g1, acc);
  }
  ksplit_reduce<kMats>(acc, red);
  if (sparts > 1 &&
      !split_sum<kMats>(acc, wid == 0, rows, p.tm,
                        p.part + (size_t)sitem * sparts * blk_floats, blk_floats, spart, sparts,
                        p.ticket + sitem))
    return;
  if (wid != 0) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = 4 * kb + j;
    if (tok < rows) {
      const float v = kPair ? silu(acc[0][j]) * acc[kMats - 1][j] : acc[0][j];
      p.out_shared[(size_t)(tok0 + tok) * Ns + nrow] = (f16)v;
    }
  }
}

template <int PHASE, int NT, int S>
static void launch_split_gm(int group_size, int blocks, const FfnArgs &a, hipStream_t st) {
  if (group_size == 64)
    hipLaunchKernelGGL((ffn_split_kernel<PHASE, NT, S, kG64>), dim3(blocks), dim3(256), 0, st, a);
  else if (group_size == 256)
    hipLaunchKernelGGL((ffn_split_kernel<PHASE, NT, S, kG256>), dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((ffn_split_kernel<PHASE, NT, S, kG128>), dim3(blocks), dim3(256), 0, st, a);
}

hipError_t launch_ffn_split(int phase, int nt, int group_size, int blocks, const FfnArgs &a,
                            hipStream_t st) {
  // the tile shapes of the whole-item launches (stages S as there)
  if (phase == 1 && nt == 1)
    launch_split_gm<1, 1, 2>(group_size, blocks, a, st);
  else if (phase == 1 && nt == 2)
    launch_split_gm<1, 2, 1>(group_size, blocks, a, st);
  else if (phase == 2 && nt == 2)
    launch_split_gm<2, 2, 2>(group_size, blocks, a, st);
  else if (phase == 2 && nt == 4)
    launch_split_gm<2, 4, 1>(group_size, blocks, a, st);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
