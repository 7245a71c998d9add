// Grouped W4 SwiGLU FFN for prefill-sized segments: a grouped GEMM on
// v_mfma_f32_32x32x16_f16 with the int4 weights dequantized in registers.
//
// Grouped GEMM over the selected experts in one launch per phase
// (xdnf.cn/news/329730 §3.2, lpnh.cn/news/2730718 §2.3); in-kernel dequant of
// the int4 expert weights, each weight unpacked once per 128-token block tile
// (the per-token re-unpacking that xdnf.cn/news/329730 §3.1 reports as
// wasteful on its GPU does not happen here).
//
// Block tile: 128 token rows (one segment tile of one expert) x 256 weight
// rows, K step 64, 4 waves.  The activation tile goes through LDS: each K
// step's 128 x 64 fp16 tile is loaded into registers one step ahead and
// stored into one of two LDS stages.  The weights do not touch LDS: wave w
// owns 64 weight rows and loads their int4 codes straight into registers
// (16 bytes per lane per 32 rows per K step, three steps ahead),
// unpacks them with the group scale folded in (RN16(q*s)) and feeds them as
// the MFMA's A operand, so every weight is read from memory and unpacked
// exactly once per block.  Each wave multiplies its 64 weight rows by all 128
// token rows: 4 x 2 accumulators of 32 x 32, holding the output transposed,
// which gives each lane 4 consecutive output columns of a token row per
// store.
//
// Phase 1 gives wave w gate rows and up rows of the same 32 ffn columns, so
// silu(g) * u is formed in registers.
//
// LDS layout of one stage: 128 rows of 128 bytes (64 halfs); the eight 16-byte
// pieces of row r are stored XOR-swizzled, piece p at position p ^ sw(r) with
// sw(r) = (r % 8) ^ ((r / 8) % 2).  The stores are 1 KB contiguous per wave
// instruction; for the MFMA operand reads (16 bytes of 16 consecutive rows
// per quarter wave) the swizzle spreads any 8 consecutive rows, and the 8
// even and the 8 odd rows of any 16, over distinct 16-byte bank groups, so
// they are free of bank conflicts whether the LDS serves 8 or 16 lanes of a
// 16-byte read per cycle.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPM = 128;          // token rows per block tile
constexpr int kPN = 256;          // weight rows per block tile
constexpr int kPK = 64;           // K per step
constexpr int kPStage = kPM * kPK;  // halfs per stage
constexpr int kPAhead = 3;        // weight codes and scales are loaded this many steps ahead

struct PrefillArgs {
  int E, H, F, T, N, k;
  const int32_t *offsets;     // [E+1]
  const int32_t *perm_src;    // phase 1 without x_perm: rows of x via perm_src[r] / k
  const f16 *a;               // phase 1: x_perm [N, H] or x [T, H]; phase 2: h [N, F]
  const uint8_t *q0, *q1;     // phase 1: gate_q, up_q; phase 2: down_q
  const f16 *s0, *s1;
  f16 *out;                   // phase 1: h [N, F]; phase 2: y_perm [N, H]
  int ntiles;                 // weight-row tiles per segment tile
  int sshift;                 // scale group of K step s: s >> sshift (group 64 / 128 / 256: 0 / 1 / 2)
};

__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The block's tile.  The routed rows of each expert are split into 128-row
// segment tiles; the (segment tile, weight-row tile) pairs are numbered in
// order and each XCD gets a contiguous run of that numbering of equal length
// (the hardware deals consecutive blocks round-robin over the 8 XCDs), so
// the blocks that share a segment tile's activations share an L2 and every
// XCD has the same amount of work.  Returns false (for the whole block) for
// blocks beyond the real number of pairs.
struct TileInfo {
  int e;          // expert
  int seg0;       // first permuted row of the segment tile
  int seg_end;    // end of the expert's segment
  int nt;         // weight-row tile
};
__device__ bool locate_tile(const int32_t *__restrict__ off, int E, int ntiles, TileInfo *t) {
  __shared__ int s_scan[4];
  __shared__ int s_res[3];
  const int tid = threadIdx.x;
  int o[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) o[i] = off[min(4 * tid + i, E)];
  int c[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = 4 * tid + i < E ? (o[i + 1] - o[i] + kPM - 1) / kPM : 0;
    sum += c[i];
  }
  int total;
  int run = block_excl_scan(sum, s_scan, &total);
  const int nvalid = total * ntiles;
  const int per_xcd = (nvalid + 7) / 8;
  const int idx = blockIdx.x / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + idx;
  if (idx >= per_xcd || logical >= nvalid) return false;
  const int slot = logical / ntiles;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (slot >= run && slot < run + c[i]) {
      s_res[0] = 4 * tid + i;
      s_res[1] = o[i] + (slot - run) * kPM;
      s_res[2] = o[i + 1];
    }
    run += c[i];
  }
  __syncthreads();
  t->e = __builtin_amdgcn_readfirstlane(s_res[0]);   // block-uniform: bases go in SGPRs
  t->seg0 = __builtin_amdgcn_readfirstlane(s_res[1]);
  t->seg_end = __builtin_amdgcn_readfirstlane(s_res[2]);
  t->nt = logical % ntiles;
  return true;
}


// Per-lane byte offsets of one block tile (step 0) and LDS offsets.
struct PrefillOperands {
  uint32_t a_off[4];          // activation pieces in the activation buffer
  int a_dst;                  // this lane's first piece in a stage (halfs)
  int a_rd[4];                // operand read offset in a stage per k16 sub-step (halfs)
  uint32_t b_off[2];          // code chunk per N-tile in its code buffer
  uint32_t s_off[2];          // group-0 scale per N-tile in its scale buffer
  int nsteps;
  int sshift;                 // scale group of step s: s >> sshift
};

// The K loop.  Step s: meet at the barrier (stage s % 2 is complete), issue
// the loads of the activation pieces of step s + 1 and of the code chunks and
// scales of step s + D (clamped to the last step; surplus loads are never
// used), run 4 k16 sub-steps of 8 MFMAs on LDS stage s % 2, then store the
// step s + 1 pieces into the other stage.  Code/scale registers rotate with
// period D + 1, hence the loop unrolled by D + 1.  MI (1..4) is the number of
// 32-row M-tiles holding real rows: the last tile of a segment skips the
// MFMAs and activation loads of its empty M-tiles (wave w loads the rows of
// M-tile w).
template <int MI, int D>
__device__ __forceinline__ void prefill_gemm(f16 *sA, rsrc_t a_rs, rsrc_t b_rs0, rsrc_t b_rs1,
                                             rsrc_t s_rs0, rsrc_t s_rs1,
                                             const PrefillOperands &o, bool a_loader,
                                             f32x16 (&acc)[MI][2]) {
  constexpr int NS = D + 1;         // code/scale register stages: steps v .. v+D
  u32x4 ra[4];                      // activation pieces of the next step
  u32x4 rb[NS][2];                  // code chunks of the steps in flight
  f16 rs[NS][2];                    // their group scales
  const int nsteps = o.nsteps;
  auto load_a = [&](int step) {
    if (!a_loader) return;
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = bload16(a_rs, o.a_off[j], step * (kPK * 2));
  };
  auto load_b = [&](int step, int u) {
    rb[u][0] = bload16(b_rs0, o.b_off[0], step * 512);
    rb[u][1] = bload16(b_rs1, o.b_off[1], step * 512);
    rs[u][0] = bload_f16(s_rs0, o.s_off[0], (step >> o.sshift) * 32);
    rs[u][1] = bload_f16(s_rs1, o.s_off[1], (step >> o.sshift) * 32);
  };
  auto store_a = [&](int step) {
    if (!a_loader) return;
    f16 *dst = sA + (step & 1) * kPStage + o.a_dst;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4 *>(dst + j * 8 * kPK) = ra[j];
  };

  const UnpackConsts kc = unpack_consts();
  // step `step` uses register stage u; the codes of step + D go to stage
  // (u + D) % NS, which held those of step - 1
  auto unpack_b = [&](int u, int w, f16x8 (&bf)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f16x8 q = unpack8(rb[u][j][w], kc);
      const f16x2 sc = {rs[u][j], rs[u][j]};
      u32x4 v;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f16x2 pr = {q[2 * t], q[2 * t + 1]};
        v[t] = as_u32(pr * sc);                    // RN16(q * s)
      }
      bf[j] = as_f16x8(v);
    }
  };
  auto read_a = [&](const f16 *as, int w, f16x8 (&af)[MI]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
      af[i] = *reinterpret_cast<const f16x8 *>(as + i * 32 * kPK + o.a_rd[w]);
  };
  // Software pipeline over the 4 k16 sub-steps: the region of sub-step w
  // holds the LDS operand reads and the weight unpack of sub-step w + 1 (for
  // w = 3: the unpack of the next step's sub-step 0, whose codes are already
  // in registers) and the MFMAs of sub-step w.  Scheduling fences keep the
  // regions apart, and inside a region scheduling groups issue the LDS reads
  // first and then one MFMA after every 4 VALU instructions, so the unpack
  // runs while the matrix core works (the counters showed half of the VALU
  // cycles without a concurrent MFMA; this order and the early unpack of the
  // next step took 1.3% off the prefill FFN).
  // bf0: the unpacked weights of the next step's first sub-step, made during
  // this step's last sub-step (its codes are in registers D steps ahead)
  f16x8 bf0[2];
  auto body = [&](int step, int u) {
    lds_barrier();      // stage step % 2 is complete; stage (step+1) % 2 is free
    const f16 *as = sA + (step & 1) * kPStage;
    f16x8 af[2][MI], bf[2][2];
    read_a(as, 0, af[0]);
    load_a(min(step + 1, nsteps - 1));
    load_b(min(step + D, nsteps - 1), (u + D) % NS);
    bf[0][0] = bf0[0];
    bf[0][1] = bf0[1];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w + 1 < 4) {
        read_a(as, w + 1, af[(w + 1) & 1]);
        unpack_b(u, w + 1, bf[(w + 1) & 1]);
      } else {
        unpack_b((u + 1) % NS, 0, bf0);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = mfma_32x32x16(bf[w & 1][j], af[w & 1][i], acc[i][j]);
      // scheduling groups (mask 0x100: LDS reads, 0x008: MFMA, 0x002: VALU)
      if (w + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, MI, 0);
#pragma unroll
      for (int g = 0; g < 2 * MI; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (step + 1 < nsteps) store_a(step + 1);
  };

  load_a(0);
#pragma unroll
  for (int u = 0; u < D; ++u) load_b(min(u, nsteps - 1), u);
  unpack_b(0, 0, bf0);
  store_a(0);
  for (int s0 = 0;; s0 += NS) {
    bool done = false;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (!done) {
        body(s0 + u, u);
        done = s0 + u + 1 >= nsteps;
      }
    }
    if (done) break;
  }
}

// Accumulate one block tile with MI live M-tiles and store it.
template <int PHASE, int MI>
__device__ __forceinline__ void prefill_tile(const PrefillArgs &p, f16 *sA, rsrc_t a_rs,
                                             rsrc_t b_rs0, rsrc_t b_rs1, rsrc_t s_rs0,
                                             rsrc_t s_rs1, const PrefillOperands &o, int seg0,
                                             int rows, int nt) {
  constexpr bool kPair = PHASE == 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int h = lane >> 5, l32 = lane & 31;
  const int Nrows = kPair ? p.F : p.H;
  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16){};
  prefill_gemm<MI, kPAhead>(sA, a_rs, b_rs0, b_rs1, s_rs0, s_rs1, o, wv < MI, acc);

  // ---- epilogue.  The weights are the MFMA's A operand, so accumulator
  // acc[i][j] holds the transposed 32 x 32 tile: register r of lane l is
  // weight row 8*(r/4) + 4*(l/32) + r%4 of N-tile j and token row l%32 of
  // M-tile i.  Registers 4q .. 4q+3 are 4 consecutive output columns of one
  // token row: one 8-byte store.
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = i * 32 + l32;
    if (m >= rows) continue;
    f16 *orow = p.out + (size_t)(seg0 + m) * Nrows;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f16 v[4];
      if (kPair) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float g = acc[i][0][4 * q + t], u = acc[i][1][4 * q + t];
          v[t] = (f16)(g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u);   // silu(g) * u
        }
        *reinterpret_cast<uint2 *>(orow + nt * 128 + wv * 32 + 8 * q + 4 * h) =
            __builtin_bit_cast(uint2, v);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = (f16)acc[i][j][4 * q + t];
          *reinterpret_cast<uint2 *>(orow + nt * kPN + wv * 64 + j * 32 + 8 * q + 4 * h) =
              __builtin_bit_cast(uint2, v);
        }
      }
    }
  }
}

template <int PHASE>
__global__ __launch_bounds__(256, 2) void ffn_prefill_kernel(PrefillArgs p) {
  constexpr bool kPair = PHASE == 1;
  __shared__ __attribute__((aligned(1024))) f16 sA[2 * kPStage];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int h = lane >> 5, l32 = lane & 31;
  const int K = kPair ? p.H : p.F;
  const int Nrows = kPair ? p.F : p.H;            // rows of one weight matrix
  const int G = (K / kPK) >> p.sshift;            // scale groups per row

  TileInfo ti;
  if (!locate_tile(p.offsets, p.E, p.ntiles, &ti)) return;
  const int e = ti.e, seg0 = ti.seg0, nt = ti.nt;
  if (seg0 < 0 || seg0 >= p.N) return;
  const int rows = min(min(kPM, ti.seg_end - seg0), p.N - seg0);

  PrefillOperands o;
  o.nsteps = K / kPK;
  o.sshift = p.sshift;
  // ---- activation pieces: piece j of wave wv's lane i is stored at row
  // r = 32*wv + 8*j + i/8, position i%8 of a stage (the wave's 64 lanes fill
  // 1 KB contiguously), which holds logical piece (i%8) ^ sw(r).  Rows past
  // the segment repeat its last row (their outputs are never stored).
  const int a_rows = p.perm_src ? p.T : p.N;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * wv + 8 * j + (lane >> 3);
    int src = seg0 + min(r, rows - 1);
    if (p.perm_src) {
      src = p.perm_src[src] / p.k;
      src = src < 0 ? 0 : (src >= p.T ? p.T - 1 : src);
    }
    o.a_off[j] = ((uint32_t)src * K + ((lane & 7) ^ (lane >> 3) ^ (j & 1)) * 8) * 2;
  }
  o.a_dst = 32 * wv * kPK + lane * 8;
  const rsrc_t a_rs = make_rsrc(p.a, (uint32_t)a_rows * K * 2);

  // ---- operand reads: for k16 sub-step w, lane l supplies row 32*i + l%32 at
  // logical piece 4*(l/32) + w, i.e. k = 32*(l/32) + 8*w .. +7 of the step
#pragma unroll
  for (int w = 0; w < 4; ++w)
    o.a_rd[w] = l32 * kPK + (((4 * h + w) ^ (lane & 7) ^ ((lane >> 3) & 1)) * 8);

  // ---- weights: N-tile j of wave wv is 32 weight rows of one matrix of
  // expert e; per step lane l loads the 16-byte chunk 2*step + l/32 of row
  // l%32, whose word w holds the same k = 32*(l/32) + 8*w .. +7 of the step
  // as the activation operand.
  const size_t mat_codes = (size_t)Nrows * (K / 2), mat_scales = (size_t)Nrows * G;
  const uint8_t *qb0 = p.q0 + (size_t)e * mat_codes;
  const uint8_t *qb1 = (kPair ? p.q1 : p.q0) + (size_t)e * mat_codes;
  const f16 *sb0 = p.s0 + (size_t)e * mat_scales;
  const f16 *sb1 = (kPair ? p.s1 : p.s0) + (size_t)e * mat_scales;
  const rsrc_t b_rs0 = make_rsrc(qb0, (uint32_t)mat_codes);
  const rsrc_t b_rs1 = make_rsrc(qb1, (uint32_t)mat_codes);
  const rsrc_t s_rs0 = make_rsrc(sb0, (uint32_t)(mat_scales * 2));
  const rsrc_t s_rs1 = make_rsrc(sb1, (uint32_t)(mat_scales * 2));
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = kPair ? nt * 128 + wv * 32 + l32 : nt * kPN + wv * 64 + j * 32 + l32;
    o.b_off[j] = (uint32_t)(n >> 4) * 8 * K + h * 256 + (n & 15) * 16;
    o.s_off[j] = ((uint32_t)(n >> 4) * 16 * G + (n & 15)) * 2;
  }

  const int mi = (rows + 31) / 32;
  if (mi >= 4)
    prefill_tile<PHASE, 4>(p, sA, a_rs, b_rs0, b_rs1, s_rs0, s_rs1, o, seg0, rows, nt);
  else if (mi == 3)
    prefill_tile<PHASE, 3>(p, sA, a_rs, b_rs0, b_rs1, s_rs0, s_rs1, o, seg0, rows, nt);
  else if (mi == 2)
    prefill_tile<PHASE, 2>(p, sA, a_rs, b_rs0, b_rs1, s_rs0, s_rs1, o, seg0, rows, nt);
  else
    prefill_tile<PHASE, 1>(p, sA, a_rs, b_rs0, b_rs1, s_rs0, s_rs1, o, seg0, rows, nt);
}

hipError_t launch_ffn_prefill_phase(const moe_layer &L, int phase, const uint16_t *a,
                                    const int32_t *perm_src, const int32_t *offsets, int32_t T,
                                    uint16_t *out, hipStream_t st) {
  const int E = L.num_experts, k = L.top_k;
  const int N = T * k;
  PrefillArgs p{};
  p.E = E; p.H = L.hidden; p.F = L.ffn; p.T = T; p.N = N; p.k = k;
  p.offsets = offsets;
  p.perm_src = perm_src;
  p.a = reinterpret_cast<const f16 *>(a);
  p.out = reinterpret_cast<f16 *>(out);
  if (phase == 1) {
    p.q0 = L.gate_q; p.q1 = L.up_q;
    p.s0 = reinterpret_cast<const f16 *>(L.gate_s);
    p.s1 = reinterpret_cast<const f16 *>(L.up_s);
    p.ntiles = L.ffn / 128;
  } else {
    p.q0 = L.down_q; p.s0 = reinterpret_cast<const f16 *>(L.down_s);
    p.ntiles = L.hidden / kPN;
  }
  p.sshift = L.group_size == 64 ? 0 : (L.group_size == 256 ? 2 : 1);
  const int max_tiles = (E < N ? E : N) + (N + kPM - 1) / kPM;
  int blocks = max_tiles * p.ntiles;
  blocks = (blocks + 7) / 8 * 8;
  if (phase == 1)
    hipLaunchKernelGGL(ffn_prefill_kernel<1>, dim3(blocks), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(ffn_prefill_kernel<2>, dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace moe
