// Host-side launchers of the gfx950 kernels (internal to libmoe_w4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe_w4.h"

namespace moe {

constexpr int kPermChunk = 256;   // flat (token, slot) entries per permutation block
// quantization group sizes the kernels implement (along in_features)
constexpr bool supported_group_size(int gs) { return gs == 64 || gs == 128 || gs == 256; }
constexpr int kFusedMaxT = 64;    // route + permute in one launch up to this many tokens
constexpr int kRouterWideMinT = 256;   // 32-token x 128-expert router tiles from this many tokens
constexpr int kFusedMaxKsb = 16;  // K parts of the fused router's logits
constexpr int kFusedMaxLogits = 8192;   // T * E held in LDS by the fused router

// The counter block at the start of every workspace (moe_workspace_init
// zero-fills it; every call leaves it at zero).
constexpr size_t kWsSyncBytes = 16384;   // a multiple of 4 KB (zero-filled by 256-thread blocks)
// Words of that block: word 0 is the one-launch router's counter; the launch
// that fuses a layer's combine with the next layer's router uses word 1 (all
// tokens) and words 32 .. 32+T-1 (one per token), hence at most 32 tokens;
// the decode FFN's K-split items take one word each from word 64 on.
constexpr int kStackAllCounter = 1;
constexpr int kStackTokCounter = 32;
constexpr int kStackMaxT = 32;
constexpr int kFfnTicket = 64;
constexpr int kFfnMaxTickets = (int)(kWsSyncBytes / 4) - kFfnTicket;

// Byte offsets of the per-call scratch regions inside the caller's workspace.
struct WsLayout {
  size_t sync;      // uint32 counters; zero between calls
  size_t logits;    // fp32 [T, E], or kFusedMaxKsb partials [T, E] when T <= kFusedMaxT,
                    // each padded to a multiple of 4 floats
  size_t counts;    // int32 [nchunks, E]
  size_t bases;     // int32 [nchunks, E]
  size_t h;         // fp16 [T*k, F]
  size_t h_shared;  // fp16 [T, Fs]
  size_t split;     // fp32 partial sums of the decode FFN's K-split blocks
  size_t total;
};
WsLayout ws_layout(const moe_layer &L, int32_t T);
// Floats of partial sums the decode FFN needs for T tokens (0: no K split).
size_t ffn_split_floats(const moe_layer &L, int32_t T);

hipError_t launch_quantize(const uint16_t *w, int64_t rows, int64_t cols, int gs, uint8_t *q,
                           uint16_t *s, hipStream_t st);
hipError_t launch_pack(const uint8_t *q_rm, const uint16_t *s_rm, int64_t rows, int64_t cols,
                       int gs, uint8_t *q, uint16_t *s, hipStream_t st);
hipError_t launch_dequant(const uint8_t *q, const uint16_t *s, int64_t rows, int64_t cols, int gs,
                          float *out, hipStream_t st);
hipError_t launch_quantize8(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *q,
                            uint16_t *s, hipStream_t st);
hipError_t launch_route(const moe_layer &L, const uint16_t *x, int32_t T, int32_t *idx,
                        float *w, float *logits, hipStream_t st);
hipError_t launch_route_permute_fused(const moe_layer &L, const uint16_t *x, int32_t T,
                                      int32_t *idx, float *w, int32_t *offsets,
                                      int32_t *perm_src, int32_t *inv_pos, float *partial,
                                      unsigned int *counter, hipStream_t st);
hipError_t launch_permute(const moe_layer &L, const uint16_t *x, const int32_t *idx, int32_t T,
                          int32_t *offsets, int32_t *perm_src, int32_t *inv_pos,
                          uint16_t *x_perm, int32_t *counts, int32_t *bases, hipStream_t st);
hipError_t launch_gather(const moe_layer &L, const uint16_t *x, const int32_t *perm_src, int32_t T,
                         uint16_t *x_perm, hipStream_t st);
// split: the workspace's partial-sum region (ffn_split_floats floats);
// tickets: its counter words from kFfnTicket on.
hipError_t launch_ffn(const moe_layer &L, const uint16_t *x, const uint16_t *x_perm,
                      const int32_t *perm_src, const int32_t *offsets, int32_t T,
                      uint16_t *y_perm, uint16_t *y_shared, uint16_t *h, uint16_t *h_shared,
                      float *split, unsigned int *tickets, hipStream_t st);
hipError_t launch_ffn_prefill_phase(const moe_layer &L, int phase, const uint16_t *a,
                                    const int32_t *perm_src, const int32_t *offsets, int32_t T,
                                    uint16_t *out, hipStream_t st);
hipError_t launch_combine(const moe_layer &L, const uint16_t *y_perm, const uint16_t *y_shared,
                          const int32_t *inv_pos, const float *w, int32_t T, uint32_t flags,
                          float eps, uint16_t *out, hipStream_t st);
// Whether a stacked decode step can fuse layer i's combine with layer i+1's
// router for T tokens of layers shaped like L.
bool stack_fused(const moe_layer &L, int32_t T);
// Layer cur's combine (flags, eps as in launch_combine) into out, then layer
// next's router, top-k and permutation on out, in one launch.  inv_pos and
// topk_w are read as layer cur's and overwritten with layer next's.
hipError_t launch_combine_route(const moe_layer &cur, const moe_layer &next,
                                const uint16_t *y_perm, const uint16_t *y_shared,
                                int32_t *inv_pos, float *topk_w, int32_t T, uint32_t flags,
                                float eps, uint16_t *out, int32_t *topk_idx, int32_t *offsets,
                                int32_t *perm_src, float *logits, unsigned int *sync,
                                hipStream_t st);

}  // namespace moe
