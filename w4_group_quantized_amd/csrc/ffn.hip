// Grouped SwiGLU expert FFN over per-expert token segments, int4 weights
// dequantized in registers right before the MFMA, plus the fp16 shared expert.
//
// Grouped GEMM over the selected experts, one launch for all of them:
// xdnf.cn/news/329730 §3.2 and lpnh.cn/news/2730718 §2.3.  Expert = gate / up /
// down matrices with a SiLU-gated product (haowenji.com/articles/
// x-2109226022155796480 §01), shared expert always on.  Decode is bound by
// streaming the selected experts' weights (lpnh.cn/news/2730718 §1.2,
// haowenji.com ... §09): every weight byte is loaded once per 16-token tile and
// unpacked once, then reused for all tokens of the tile on the matrix cores.
//
// Phase 1 (gate/up):  h[r] = silu(deq(Wg_e) x[r]) * (deq(Wu_e) x[r])  -> fp16
// Phase 2 (down):     y[r] = deq(Wd_e) h[r]                          -> fp16
// The phases are separate launches because phase 2 of an expert needs every
// column of h for its rows.
//
// Work items (one 256-thread block each; the shared-expert items come first,
// so they start with the first wave of blocks instead of waiting for slots
// behind the routed ones):
//   routed item = (segment tile, n-tile): a segment tile is 16 consecutive rows
//     of one expert's segment; an n-tile is 64*NT weight rows; each of the 4
//     waves streams 16*NT rows over the whole K range.  When the tile's live
//     token rows fit in 32 KB the block stages them in LDS once and the waves
//     read their MFMA operands from there.
//   shared item = (16-token tile, 16 weight rows); the 4 waves split K 4 ways,
//     so that a wave moves as many bytes as a routed wave (fp16 weights are 4x
//     the bytes of int4).  The shared expert's weights are fp16, or 8-bit g128
//     codes (xdnf.cn/news/329730 §3.1 keeps the shared FFN at 8 bits).
// The grid is sized for the worst case on the host; items past the live
// segment tiles exit right after locating themselves (nothing is read back to
// the host between calls).
//
// Batches of a few tokens whose items would leave some CUs streaming two of
// them while others idle after one split each item's K range over several
// blocks (the host's rule is with launch_ffn), so that every CU streams about
// the same number of bytes: a CU reads ~20 GB/s whether it holds one block or
// three.  The item's last block to finish adds the fp32 partial sums of its
// parts in the fixed order 0, 1, ..., P-1.
#include "ffn_decode.h"

namespace moe {

// PHASE 1: PAIR = gate and up tiles per wave, SwiGLU epilogue.
// PHASE 2: one matrix, plain epilogue.  GM: quantization group size (GroupMode).
// STREAM: code loads streamed past the caches (see launch_ffn).
template <int PHASE, int NT, int S, int GM, bool STREAM>
__global__ __launch_bounds__(256) void ffn_decode_kernel(FfnArgs p) {
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

  if ((int)blockIdx.x >= p.shared_items) {
    const int item = blockIdx.x - p.shared_items;
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
      w4_tiles<kMats * NT, S, GM, STREAM>(al, qrow, srow, 0, G, acc, [&] {
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
      w4_tiles<kMats * NT, S, GM, STREAM>(arow, qrow, srow, 0, G, acc);
    }
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

  // shared expert: fp16 weights, 16 weight rows per block, K split over waves
  const int Ks = kPair ? p.H : p.Fs;
  const int Ns = kPair ? p.Fs : p.H;
  const int Gs = Ks / kGroup;
  const int sitem = blockIdx.x;
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
  const int g0 = wid * Gs / 4, g1 = (wid + 1) * Gs / 4;
  if (p.shared_w8) {     // block-uniform: 8-bit codes, 16-row tile nt
    const size_t tile = (size_t)nt * 16;
    const uint8_t *qrow[kMats];
    const f16 *srow[kMats];
    qrow[0] = p.wq0 + tile * Ks + kb * 512 + r * 16;
    srow[0] = p.ws0 + tile * Gs + r;
    if (kPair) {
      qrow[kMats - 1] = p.wq1 + tile * Ks + kb * 512 + r * 16;
      srow[kMats - 1] = p.ws1 + tile * Gs + r;
    }
    w8_tiles<kMats, STREAM>(arow, qrow, srow, g0, g1, acc);
  } else {
    const f16 *wrow[kMats];
    wrow[0] = p.w0 + (size_t)nrow * Ks;
    if (kPair) wrow[kMats - 1] = p.w1 + (size_t)nrow * Ks;
    f16_tiles<kMats>(arow, wrow, kb, g0, g1, acc);
  }
  ksplit_reduce<kMats>(acc, red);
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

// Tile shapes per phase.  Rows per block = 64 * NT (each wave streams NT
// 16-row tiles of each matrix); S = quantization groups per pipeline stage.
// Small segments (under kWideMinAvgRows rows per expert on average, so the
// token rows come from LDS): gate/up NT 1, S 2; down NT 2, S 2.  Segments of
// several rows: NT 2, S 1 for gate/up and NT 4, S 1 for down, so that each
// activation load serves more weight bytes.
constexpr int kWideMinAvgRows = 2;

// Prefill mode: segments average at least this many rows, so a 128-row MFMA
// block tile is mostly full; routed experts then run on the MFMA kernel.  Its
// buffer loads address each activation matrix and each expert's weight
// matrix with 32-bit byte offsets.
constexpr int kPrefillMinAvgRows = 32;

// One decode launch, instantiated for the layer's group size.
template <int PHASE, int NT, int S, bool STREAM>
static void launch_decode(int group_size, int blocks, const FfnArgs &a, hipStream_t st) {
  if (group_size == 64)
    hipLaunchKernelGGL((ffn_decode_kernel<PHASE, NT, S, kG64, STREAM>), dim3(blocks), dim3(256),
                       0, st, a);
  else if (group_size == 256)
    hipLaunchKernelGGL((ffn_decode_kernel<PHASE, NT, S, kG256, STREAM>), dim3(blocks), dim3(256),
                       0, st, a);
  else
    hipLaunchKernelGGL((ffn_decode_kernel<PHASE, NT, S, kG128, STREAM>), dim3(blocks), dim3(256),
                       0, st, a);
}

bool ffn_prefill_mode(const moe_layer &L, int32_t T) {
  const int64_t N = (int64_t)T * L.top_k;
  const int64_t H = L.hidden, F = L.ffn;
  const int64_t max_bytes = int64_t(1) << 31;
  return N >= (int64_t)kPrefillMinAvgRows * L.num_experts && H % 256 == 0 &&
         N * H * 2 < max_bytes && N * F * 2 < max_bytes && F * H / 2 < max_bytes;
}

// The decode launches of a layer at T tokens: tile shapes, worst-case item
// counts and K parts of the two phases.
struct DecodePlan {
  bool prefill, wide, stream, wide2;
  int routed1, shared1, routed2, shared2;   // items
  int rparts1, sparts1, rparts2, sparts2;   // blocks per item
  int tm;                                   // token rows per tile in the partial sums
};

static DecodePlan decode_plan(const moe_layer &L, int32_t T) {
  DecodePlan d{};
  const int64_t E = L.num_experts, H = L.hidden, F = L.ffn, Fs = L.shared_ffn, k = L.top_k;
  const int64_t N = (int64_t)T * k;
  d.prefill = ffn_prefill_mode(L, T);
  // worst case number of 16-row segment tiles: every non-empty segment adds at
  // most one partial tile
  const int64_t max_tiles = (E < N ? E : N) + (N + kTileM - 1) / kTileM;
  const int64_t mtiles_shared = (T + kTileM - 1) / kTileM;
  d.wide = N >= kWideMinAvgRows * E;
  // Code loads are streamed past the caches unless a segment can span several
  // 16-row tiles (T > 16) that all read the expert's weights and the segments
  // are long on average (the wide shapes): measured on the 288-expert layer,
  // streaming is 9% / 4% / 1.4% faster at 8 / 32 / 64 tokens, caching 2.4%
  // faster at 150 tokens; a layer with T <= 16 never reads a weight twice.
  d.stream = T <= kTileM || !d.wide;
  // Down tiles of 256 rows (NT 4) also when its K, the ffn width, is short:
  // at 640 columns (5 groups) per row the 128-row shape's blocks are mostly
  // start-up (measured on the 512-expert layer: 37.0-37.6 against 37.9 us
  // per FFN call; at 1536 columns the 128-row shape stays 1.5% faster).
  d.wide2 = (d.wide || F <= 1024) && H % 256 == 0;
  const int nt1 = d.wide ? 2 : 1, nt2 = d.wide2 ? 4 : 2;
  d.routed1 = d.prefill ? 0 : (int)(max_tiles * (F / (64 * nt1)));   // F % 128 == 0
  d.shared1 = Fs ? (int)(mtiles_shared * (Fs / 16)) : 0;
  d.routed2 = d.prefill ? 0 : (int)(max_tiles * (H / (64 * nt2)));   // H % 128 == 0
  d.shared2 = Fs ? (int)(mtiles_shared * (H / 16)) : 0;
  d.rparts1 = d.sparts1 = d.rparts2 = d.sparts2 = 1;
  d.tm = T < kTileM ? (T > 0 ? T : 1) : kTileM;
  // (a split launch is a streamed one: only those have a split instance; the
  // 8-bit shared expert is never split: at one token on the 288-expert layer
  // the split the rule would pick measured 2-5% slower, and the split kernel
  // has no 8-bit path)
  if (d.prefill || T > kSplitMaxT || !d.stream || (Fs > 0 && L.shared_bits == 8)) return d;
  // Routed items that can be live: with T <= 16 every segment is one tile, so
  // at most min(E, N) tiles (the grid's last items exit on locating
  // themselves), and split blocks index their partial sums among those.
  const int64_t live = E < N ? E : N;
  const int64_t sh_elem = L.shared_bits == 8 ? 1 : 2;
  auto plan_phase = [&](int64_t K, int64_t Ks, int nt, int kmats, int routed, int shared,
                        int slots, int *rp, int *sp) {
    const int64_t rb = 64 * nt * kmats * (K / 2 + K / L.group_size * 2);   // codes + scales
    const int64_t sb = 16 * kmats * Ks * sh_elem;
    const int64_t nr = live * (routed / max_tiles);
    // at least two quantization groups per routed block and per shared wave
    split_parts(nr, rb, (int)(K / kGroup / 2), shared, sb, (int)(Ks / kGroup / 8), slots, rp, sp);
    if ((int64_t)routed + shared > kFfnMaxTickets ||
        (size_t)(nr * *rp + (int64_t)shared * *sp) * 4 * nt * kmats * d.tm * 16 >
            split_floats(slots, nt * kmats, d.tm))
      *rp = *sp = 1;
  };
  plan_phase(H, H, nt1, 2, d.routed1, d.shared1, 3, &d.rparts1, &d.sparts1);
  plan_phase(F, Fs, nt2, 1, d.routed2, d.shared2, nt2 == 4 ? 4 : 3, &d.rparts2, &d.sparts2);
  return d;
}

size_t ffn_split_floats(const moe_layer &L, int32_t T) {
  // The largest need of any batch up to T tokens, so that a workspace sized
  // for T tokens serves every smaller batch.  It depends on neither the group
  // size nor the shared expert's format, so one workspace serves every layer
  // of a stack whose layers agree in experts, widths and top-k.
  // A phase whose items stay under two kSplitMinBytes blocks even at the
  // largest (64-wide groups, fp16 shared expert) never splits.
  const int64_t H = L.hidden, F = L.ffn, Fs = L.shared_ffn;
  auto can_split = [](int64_t K, int64_t Ks, int nt, int kmats) {
    const int64_t rb = 64 * nt * kmats * (K / 2 + K / 32), sb = 16 * kmats * Ks * 2;
    return rb >= 2 * kSplitMinBytes || sb >= 2 * kSplitMinBytes;
  };
  size_t m = 0;
  for (int32_t t = 1; t <= T && t <= kSplitMaxT; ++t) {
    if (ffn_prefill_mode(L, t)) continue;
    const int64_t N = (int64_t)t * L.top_k;
    const bool wide = N >= kWideMinAvgRows * L.num_experts;     // as decode_plan
    const bool wide2 = (wide || F <= 1024) && H % 256 == 0;
    const int nt1 = wide ? 2 : 1, nt2 = wide2 ? 4 : 2;
    const size_t f1 = can_split(H, H, nt1, 2) ? split_floats(3, 2 * nt1, t) : 0;
    const size_t f2 = can_split(F, Fs, nt2, 1) ? split_floats(nt2 == 4 ? 4 : 3, nt2, t) : 0;
    m = f1 > m ? f1 : m;
    m = f2 > m ? f2 : m;
  }
  return m;
}

hipError_t launch_ffn(const moe_layer &L, const uint16_t *x, const uint16_t *x_perm,
                      const int32_t *perm_src, const int32_t *offsets, int32_t T,
                      uint16_t *y_perm, uint16_t *y_shared, uint16_t *h, uint16_t *h_shared,
                      float *split, unsigned int *tickets, hipStream_t st) {
  const int E = L.num_experts, H = L.hidden, F = L.ffn, Fs = L.shared_ffn, k = L.top_k;
  const int N = T * k;
  const DecodePlan d = decode_plan(L, T);

  FfnArgs a{};
  a.E = E; a.H = H; a.F = F; a.Fs = Fs; a.T = T; a.N = N; a.k = k;
  a.offsets = offsets;
  a.tm = d.tm;
  a.part = split;
  a.ticket = tickets;

  // phase 1: token rows from x_perm, or from x through perm_src
  hipError_t err = hipSuccess;
  if (d.prefill) {
    err = launch_ffn_prefill_phase(L, 1, x_perm ? x_perm : x, x_perm ? nullptr : perm_src,
                                   offsets, T, h, st);
    if (err != hipSuccess) return err;
  }
  a.perm_src = x_perm ? nullptr : perm_src;
  a.a_routed = reinterpret_cast<const f16 *>(x_perm ? x_perm : x);
  a.a_shared = reinterpret_cast<const f16 *>(x);
  a.q0 = L.gate_q; a.q1 = L.up_q;
  a.s0 = reinterpret_cast<const f16 *>(L.gate_s);
  a.s1 = reinterpret_cast<const f16 *>(L.up_s);
  a.w0 = reinterpret_cast<const f16 *>(L.shared_gate);
  a.w1 = reinterpret_cast<const f16 *>(L.shared_up);
  a.shared_w8 = L.shared_bits == 8;
  a.wq0 = L.shared_gate_q; a.wq1 = L.shared_up_q;
  a.ws0 = reinterpret_cast<const f16 *>(L.shared_gate_s);
  a.ws1 = reinterpret_cast<const f16 *>(L.shared_up_s);
  a.out_routed = reinterpret_cast<f16 *>(h);
  a.out_shared = reinterpret_cast<f16 *>(h_shared);
  a.routed_items = d.routed1;
  a.shared_items = d.shared1;
  a.rparts = d.rparts1;
  a.sparts = d.sparts1;
  int blocks = a.routed_items * a.rparts + a.shared_items * a.sparts;
  if (blocks > 0) {
    if (a.rparts > 1 || a.sparts > 1)   // split launches are streamed ones
      err = launch_ffn_split(1, d.wide ? 2 : 1, L.group_size, blocks, a, st);
    else if (d.wide && d.stream)
      launch_decode<1, 2, 1, true>(L.group_size, blocks, a, st);
    else if (d.wide)
      launch_decode<1, 2, 1, false>(L.group_size, blocks, a, st);
    else
      launch_decode<1, 1, 2, true>(L.group_size, blocks, a, st);
    if (err != hipSuccess || (err = hipGetLastError()) != hipSuccess) return err;
  }

  // phase 2
  if (d.prefill) {
    err = launch_ffn_prefill_phase(L, 2, h, nullptr, offsets, T, y_perm, st);
    if (err != hipSuccess) return err;
  }
  a.perm_src = nullptr;
  a.a_routed = reinterpret_cast<const f16 *>(h);
  a.a_shared = reinterpret_cast<const f16 *>(h_shared);
  a.q0 = L.down_q; a.q1 = nullptr;
  a.s0 = reinterpret_cast<const f16 *>(L.down_s); a.s1 = nullptr;
  a.w0 = reinterpret_cast<const f16 *>(L.shared_down); a.w1 = nullptr;
  a.wq0 = L.shared_down_q; a.wq1 = nullptr;
  a.ws0 = reinterpret_cast<const f16 *>(L.shared_down_s); a.ws1 = nullptr;
  a.out_routed = reinterpret_cast<f16 *>(y_perm);
  a.out_shared = reinterpret_cast<f16 *>(y_shared);
  a.routed_items = d.routed2;
  a.shared_items = d.shared2;
  a.rparts = d.rparts2;
  a.sparts = d.sparts2;
  blocks = a.routed_items * a.rparts + a.shared_items * a.sparts;
  if (blocks > 0) {
    if (a.rparts > 1 || a.sparts > 1)
      err = launch_ffn_split(2, d.wide2 ? 4 : 2, L.group_size, blocks, a, st);
    else if (d.wide2 && d.stream)
      launch_decode<2, 4, 1, true>(L.group_size, blocks, a, st);
    else if (d.wide2)
      launch_decode<2, 4, 1, false>(L.group_size, blocks, a, st);
    else if (d.stream)
      launch_decode<2, 2, 2, true>(L.group_size, blocks, a, st);
    else
      launch_decode<2, 2, 2, false>(L.group_size, blocks, a, st);
    if (err != hipSuccess || (err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
