// Grouped W4 SwiGLU FFN for prefill-sized segments: an LDS-tiled grouped GEMM
// on v_mfma_f32_32x32x16_f16.
//
// Grouped GEMM over the selected experts in one launch per phase
// (xdnf.cn/news/329730 §3.2, lpnh.cn/news/2730718 §2.3); in-kernel dequant of
// the int4 expert weights, unpacked once per block tile and reused by every
// token row of the tile (the per-token re-unpacking that xdnf.cn/news/329730
// §3.1 reports as wasteful on its GPU does not happen here).
//
// Block tile: 128 token rows (one segment tile of one expert) x 256 weight
// rows, K step 32.  Per K step the block loads the 256 x 32 int4 codes
// (16 bytes per thread, one 256-byte chunk per 16-row tile of the storage
// layout) and the 128 x 32 fp16 activations, dequantizes the codes with their
// group scale into fp16 (RN16(q*s)) and writes both into one of two LDS
// buffers; the 4 waves (2 x 2) each multiply a 64 x 128 sub-tile with 8
// 32x32 accumulators while the next K step's global loads are in flight.
// Phase 1 orders the 256 B rows as [gate f0..63 | up f0..63 | gate f64..127
// | up f64..127] so each wave holds matching gate and up columns and applies
// silu(g) * u in registers.
#include "common.h"
#include "kernels.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPM = 128;          // token rows per block tile
constexpr int kPN = 256;          // weight rows per block tile
constexpr int kPK = 32;           // K per step
constexpr int kPLda = kPK + 8;    // LDS row stride in halfs (padding against bank conflicts)

struct PrefillArgs {
  int E, H, F, T, N, k;
  const int32_t *offsets;     // [E+1]
  const int32_t *perm_src;    // phase 1 without x_perm: rows of x via perm_src[r] / k
  const f16 *a;               // phase 1: x_perm [N, H] or x [T, H]; phase 2: h [N, F]
  const uint8_t *q0, *q1;     // phase 1: gate_q, up_q; phase 2: down_q
  const f16 *s0, *s1;
  f16 *out;                   // phase 1: h [N, F]; phase 2: y_perm [N, H]
  int ntiles;                 // weight-row tiles per segment tile
  int nblocks;                // grid size (a multiple of 8)
};

__device__ __forceinline__ f32x16 mfma_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Which expert and which 128-row tile of its segment is segment tile `slot`?
__device__ bool locate_tile128(const int32_t *__restrict__ off, int E, int slot, int *e_out,
                               int *mt_out) {
  __shared__ int s_scan[4];
  __shared__ int s_res[2];
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

template <int PHASE>
__global__ __launch_bounds__(256, 2) void ffn_prefill_kernel(PrefillArgs p) {
  constexpr bool kPair = PHASE == 1;
  __shared__ __attribute__((aligned(16))) f16 sA[2][kPM * kPLda];
  __shared__ __attribute__((aligned(16))) f16 sB[2][kPN * kPLda];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int wm = wid >> 1, wn = wid & 1;          // 2 x 2 waves: 64 rows x 128 cols each
  const int K = kPair ? p.H : p.F;
  const int Nrows = kPair ? p.F : p.H;            // rows of one weight matrix
  const int G = K / kGroup;

  // XCD-aware order: hardware round-robins consecutive blocks over the 8
  // XCDs; give each XCD a contiguous run of logical tiles so the blocks that
  // share a segment tile's activations share an L2.
  const int per_xcd = p.nblocks / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int slot = logical / p.ntiles, nt = logical % p.ntiles;
  int e, mt;
  if (!locate_tile128(p.offsets, p.E, slot, &e, &mt)) return;
  const int seg0 = p.offsets[e] + mt * kPM;
  if (seg0 < 0 || seg0 >= p.N) return;
  const int rows = min(min(kPM, p.offsets[e + 1] - seg0), p.N - seg0);

  // ---- loader assignments
  // A: thread -> token row tid/2, 16 halfs at k offset (tid&1)*16
  const int a_row = tid >> 1, a_k = (tid & 1) * 16;
  int a_src = seg0 + min(a_row, rows - 1);
  if (p.perm_src) {
    a_src = p.perm_src[a_src] / p.k;
    a_src = a_src < 0 ? 0 : (a_src >= p.T ? p.T - 1 : a_src);
  }
  const f16 *a_ptr = p.a + (size_t)a_src * K + a_k;
  // B: thread -> 16-row storage tile tt = tid/16, row r = tid%16; 16 bytes
  // (32 codes) of chunk (4g + step) per K step
  const int tt = tid >> 4, br = tid & 15;
  int b_lds_row, w_row;
  const uint8_t *qbase;
  const f16 *sbase;
  if (kPair) {
    const int mat = (tt >> 2) & 1;                 // 0 gate, 1 up
    const int ftile = (tt >> 3) * 4 + (tt & 3);    // 16-row tile among the 128 f values
    w_row = nt * 128 + ftile * 16;                 // first row of the storage tile
    b_lds_row = ((tt >> 3) * 128) + mat * 64 + (tt & 3) * 16 + br;
    qbase = mat ? p.q1 : p.q0;
    sbase = mat ? p.s1 : p.s0;
  } else {
    w_row = nt * kPN + tt * 16;
    b_lds_row = tt * 16 + br;
    qbase = p.q0;
    sbase = p.s0;
  }
  const size_t mat_row0 = (size_t)e * Nrows + w_row;
  const uint8_t *b_ptr = qbase + mat_row0 * (K / 2) + br * 16;   // + chunk * 256
  const f16 *s_ptr = sbase + mat_row0 * G + br;                   // + g * 16

  const UnpackConsts kc = unpack_consts();
  const int nsteps = K / kPK;

  u32x4 ra0, ra1, rb;
  f16 rs;
  auto gload = [&](int step) {
    const int k0 = step * kPK;
    ra0 = ld16(a_ptr + k0);
    ra1 = ld16(a_ptr + k0 + 8);
    rb = ld16(b_ptr + (size_t)step * 256);     // chunk index = step (4 chunks per group)
    rs = s_ptr[(size_t)(step >> 2) * 16];
  };
  auto lstore = [&](int buf) {
    *reinterpret_cast<u32x4 *>(&sA[buf][a_row * kPLda + a_k]) = ra0;
    *reinterpret_cast<u32x4 *>(&sA[buf][a_row * kPLda + a_k + 8]) = ra1;
    const f16x2 sc = {rs, rs};
    f16 *dst = &sB[buf][b_lds_row * kPLda];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      f16x8 c = unpack8(rb[w], kc);
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 pr = {c[2 * j], c[2 * j + 1]};
        o[j] = as_u32(pr * sc);                    // RN16(q * s)
      }
      *reinterpret_cast<u32x4 *>(dst + w * 8) = o;
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};

  gload(0);
  lstore(0);
  __syncthreads();
  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) gload(step + 1);
#pragma unroll
    for (int ks = 0; ks < kPK; ks += 16) {
      f16x8 af[2], bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const f16x8 *>(
            &sA[buf][(wm * 64 + i * 32 + lrow) * kPLda + ks + lk]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const f16x8 *>(
            &sB[buf][(wn * 128 + j * 32 + lrow) * kPLda + ks + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16(af[i], bf[j], acc[i][j]);
    }
    if (step + 1 < nsteps) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: D register r of lane l is row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32 of its 32x32 tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= rows) continue;
      f16 *orow = p.out + (size_t)(seg0 + m) * Nrows;
      if (kPair) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float g = acc[i][j][r], u = acc[i][j + 2][r];
          const int f = nt * 128 + wn * 64 + j * 32 + (lane & 31);
          orow[f] = (f16)(g / (1.0f + expf(-g)) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) orow[nt * kPN + wn * 128 + j * 32 + (lane & 31)] = (f16)acc[i][j][r];
      }
    }
  }
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
  const int max_tiles = (E < N ? E : N) + (N + kPM - 1) / kPM;
  int blocks = max_tiles * p.ntiles;
  blocks = (blocks + 7) / 8 * 8;
  p.nblocks = blocks;
  if (phase == 1)
    hipLaunchKernelGGL(ffn_prefill_kernel<1>, dim3(blocks), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(ffn_prefill_kernel<2>, dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace moe
