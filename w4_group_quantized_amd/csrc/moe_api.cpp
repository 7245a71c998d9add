// C ABI of libmoe_w4: argument checks on the host, workspace carving, and the
// launches.  Nothing here allocates, frees or synchronizes.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stddef.h>

#include <mutex>

#include "../../include/moe_w4.h"
#include "common.h"
#include "kernels.h"

namespace moe {

static inline size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

static inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static inline bool ok_ptr(const void *p) { return p != nullptr && aligned16(p); }

WsLayout ws_layout(const moe_layer &L, int32_t T) {
  WsLayout w{};
  const size_t Tz = (size_t)(T > 0 ? T : 0);
  const size_t E = (size_t)L.num_experts, k = (size_t)L.top_k;
  const size_t N = Tz * k;
  const size_t nch = (N + kPermChunk - 1) / kPermChunk;
  size_t off = 0;
  w.sync = off;     off += kWsSyncBytes;
  const bool fused = Tz <= (size_t)kFusedMaxT && Tz * E <= (size_t)kFusedMaxLogits;
  // the fused router's K parts each padded to a multiple of 4 logits
  const size_t nlog = fused ? (size_t)kFusedMaxKsb * ((Tz * E + 3) & ~(size_t)3) : Tz * E;
  w.logits = off;   off += align_up(nlog * sizeof(float));
  w.counts = off;   off += align_up(nch * E * sizeof(int32_t));
  w.bases = off;    off += align_up(nch * E * sizeof(int32_t));
  w.h = off;        off += align_up(N * (size_t)L.ffn * 2);
  w.h_shared = off; off += align_up(Tz * (size_t)L.shared_ffn * 2);
  w.split = off;    off += align_up(ffn_split_floats(L, (int32_t)Tz) * sizeof(float));
  w.total = off;
  return w;
}

// Shape limits of the kernels.
static moe_status check_layer(const moe_layer *L) {
  if (!L) return MOE_EINVAL;
  if (!supported_group_size(L->group_size)) return MOE_EUNSUPPORTED;
  if (L->num_experts < 1 || L->num_experts > 1024) return MOE_EUNSUPPORTED;
  if (L->hidden < 128 || L->hidden > 65536 || L->hidden % 128) return MOE_EUNSUPPORTED;
  if (L->ffn < 128 || L->ffn > 262144 || L->ffn % 128) return MOE_EUNSUPPORTED;
  if (L->top_k < 1 || L->top_k > 32 || L->top_k > L->num_experts) return MOE_EUNSUPPORTED;
  if (L->shared_ffn < 0 || L->shared_ffn > 262144 || L->shared_ffn % 128)
    return MOE_EUNSUPPORTED;
  // whole groups per row of every int4 matrix (in_features H and F)
  if (L->hidden % L->group_size || L->ffn % L->group_size) return MOE_EUNSUPPORTED;
  if (L->shared_bits != 0 && L->shared_bits != 16 && L->shared_bits != 8) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static moe_status check_tokens(const moe_layer *L, int32_t T) {
  if (T < 0) return MOE_EINVAL;
  // every flat index and every element offset of the permuted rows must fit
  if ((int64_t)T * L->top_k > (int64_t)0x7fffffff / 2) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

static moe_status check_ws(const moe_layer *L, int32_t T, const void *ws, size_t ws_bytes) {
  const size_t need = ws_layout(*L, T).total;
  if (need && !ok_ptr(ws)) return MOE_EINVAL;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  return MOE_OK;
}

// The HIP error behind the last MOE_EHIP returned on this thread.
static thread_local hipError_t g_last_hip_error = hipSuccess;

static inline moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = e;
  return MOE_EHIP;
}

// Errors left behind by earlier HIP calls of other code on this thread must
// not be reported as ours: clear them before launching.
static inline void clear_stale_hip_error() { (void)hipGetLastError(); }

// Pointer checks of the stages (the layer and T > 0 already checked).
static moe_status check_route_args(const moe_layer *L, const uint16_t *x,
                                   const int32_t *topk_idx, const float *topk_w) {
  if (!ok_ptr(L->router_w) || !ok_ptr(x) || !ok_ptr(topk_idx) || !ok_ptr(topk_w))
    return MOE_EINVAL;
  if (L->router_b && !aligned16(L->router_b)) return MOE_EINVAL;
  return MOE_OK;
}

static moe_status check_permute_args(const uint16_t *x, const int32_t *topk_idx,
                                     const int32_t *offsets, const int32_t *perm_src,
                                     const int32_t *inv_pos, const uint16_t *x_perm) {
  if (!ok_ptr(topk_idx) || !ok_ptr(offsets) || !ok_ptr(perm_src) || !ok_ptr(inv_pos))
    return MOE_EINVAL;
  if (x_perm && (!ok_ptr(x) || !aligned16(x_perm))) return MOE_EINVAL;
  return MOE_OK;
}

static moe_status check_ffn_args(const moe_layer *L, int32_t T, const uint16_t *x,
                                 const uint16_t *x_perm, const int32_t *perm_src,
                                 const int32_t *offsets, const uint16_t *y_perm,
                                 const uint16_t *y_shared) {
  if (!ok_ptr(offsets) || !ok_ptr(y_perm) || !ok_ptr(L->gate_q) || !ok_ptr(L->gate_s) ||
      !ok_ptr(L->up_q) || !ok_ptr(L->up_s) || !ok_ptr(L->down_q) || !ok_ptr(L->down_s))
    return MOE_EINVAL;
  if (x_perm ? !aligned16(x_perm) : (!ok_ptr(x) || !ok_ptr(perm_src))) return MOE_EINVAL;
  // gathering rows straight from x addresses it with 32-bit byte offsets
  if (!x_perm && (int64_t)T * L->hidden * 2 >= ((int64_t)1 << 31)) return MOE_EUNSUPPORTED;
  if (L->shared_ffn > 0) {
    if (!ok_ptr(x) || !ok_ptr(y_shared)) return MOE_EINVAL;
    if (L->shared_bits == 8) {
      if (!ok_ptr(L->shared_gate_q) || !ok_ptr(L->shared_gate_s) || !ok_ptr(L->shared_up_q) ||
          !ok_ptr(L->shared_up_s) || !ok_ptr(L->shared_down_q) || !ok_ptr(L->shared_down_s))
        return MOE_EINVAL;
    } else if (!ok_ptr(L->shared_gate) || !ok_ptr(L->shared_up) || !ok_ptr(L->shared_down)) {
      return MOE_EINVAL;
    }
  }
  return MOE_OK;
}

static moe_status check_combine_args(const uint16_t *y_perm, const uint16_t *y_shared,
                                     const int32_t *inv_pos, const float *topk_w,
                                     uint32_t flags, float eps, const uint16_t *out) {
  if (!ok_ptr(y_perm) || !ok_ptr(inv_pos) || !ok_ptr(topk_w) || !ok_ptr(out)) return MOE_EINVAL;
  if (y_shared && !aligned16(y_shared)) return MOE_EINVAL;
  if (flags & ~(MOE_RMSNORM | MOE_RENORM)) return MOE_EINVAL;
  if ((flags & MOE_RMSNORM) && !(eps >= 0.0f)) return MOE_EINVAL;
  return MOE_OK;
}

// Zero-fills n 16-byte words (a kernel, not a memset node, so that the call
// can sit in a captured graph).
__global__ __launch_bounds__(256) void zero_words_kernel(u32x4 *p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = (u32x4){0u, 0u, 0u, 0u};
}

// The decode FFN's per-item tickets in the workspace's counter block.
static inline unsigned int *ffn_tickets(char *base, const WsLayout &w) {
  return reinterpret_cast<unsigned int *>(base + w.sync) + kFfnTicket;
}

static inline bool fused_route(const moe_layer &L, int32_t T) {
  return T <= kFusedMaxT && (int64_t)T * L.num_experts <= kFusedMaxLogits;
}

// Route + permute on `st`: one launch for small batches, else the router
// and the permutation launches.
static hipError_t run_route_permute(const moe_layer &L, const uint16_t *x, int32_t T,
                                    int32_t *topk_idx, float *topk_w, int32_t *offsets,
                                    int32_t *perm_src, int32_t *inv_pos, uint16_t *x_perm,
                                    char *base, const WsLayout &w, hipStream_t st) {
  if (fused_route(L, T)) {
    hipError_t e = launch_route_permute_fused(
        L, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos,
        reinterpret_cast<float *>(base + w.logits), reinterpret_cast<unsigned int *>(base + w.sync),
        st);
    if (e == hipSuccess && x_perm) e = launch_gather(L, x, perm_src, T, x_perm, st);
    return e;
  }
  hipError_t e = launch_route(L, x, T, topk_idx, topk_w,
                              reinterpret_cast<float *>(base + w.logits), st);
  if (e == hipSuccess)
    e = launch_permute(L, x, topk_idx, T, offsets, perm_src, inv_pos, x_perm,
                       reinterpret_cast<int32_t *>(base + w.counts),
                       reinterpret_cast<int32_t *>(base + w.bases), st);
  return e;
}

// The whole layer on `st` with a prepared workspace of ws_bytes at `base`;
// every argument already checked.
static moe_status run_layer(const moe_layer &L, const uint16_t *x, int32_t T, int32_t *topk_idx,
                            float *topk_w, int32_t *offsets, int32_t *perm_src, int32_t *inv_pos,
                            uint16_t *x_perm, uint16_t *y_perm, uint16_t *ys, uint32_t flags,
                            float eps, uint16_t *out, char *base, hipStream_t st) {
  const WsLayout w = ws_layout(L, T);
  hipError_t e = run_route_permute(L, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm,
                                   base, w, st);
  if (e == hipSuccess)
    e = launch_ffn(L, x, x_perm, perm_src, offsets, T, y_perm, ys,
                   reinterpret_cast<uint16_t *>(base + w.h),
                   reinterpret_cast<uint16_t *>(base + w.h_shared),
                   reinterpret_cast<float *>(base + w.split), ffn_tickets(base, w), st);
  if (e == hipSuccess)
    e = launch_combine(L, y_perm, ys, inv_pos, topk_w, T, flags, eps, out, st);
  return hip_status(e);
}

// A decode step through n stacked layers of one shape on `st` (arguments
// checked): layer i reads in_i (x, then the previous layer's output) and
// writes acts[i].  When stack_fused allows, layer i's combine and layer i+1's
// routing share one launch; otherwise each layer runs as run_layer does.
static moe_status run_stack(const moe_layer *const *layers, int32_t n, const uint16_t *x,
                            int32_t T, int32_t *topk_idx, float *topk_w, int32_t *offsets,
                            int32_t *perm_src, int32_t *inv_pos, uint16_t *y_perm, uint16_t *ys,
                            uint32_t flags, float eps, uint16_t *acts, char *base,
                            hipStream_t st) {
  const moe_layer &L0 = *layers[0];
  const WsLayout w = ws_layout(L0, T);
  const size_t HT = (size_t)T * (size_t)L0.hidden;
  const bool fused = stack_fused(L0, T);
  uint16_t *h = reinterpret_cast<uint16_t *>(base + w.h);
  uint16_t *hs = reinterpret_cast<uint16_t *>(base + w.h_shared);
  hipError_t e = run_route_permute(L0, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos,
                                   nullptr, base, w, st);
  const uint16_t *in = x;
  for (int32_t i = 0; i < n && e == hipSuccess; ++i) {
    const moe_layer &L = *layers[i];
    uint16_t *out = acts + (size_t)i * HT;
    e = launch_ffn(L, in, nullptr, perm_src, offsets, T, y_perm, ys, h, hs,
                   reinterpret_cast<float *>(base + w.split), ffn_tickets(base, w), st);
    if (e != hipSuccess) break;
    if (fused && i + 1 < n) {
      e = launch_combine_route(L, *layers[i + 1], y_perm, ys, inv_pos, topk_w, T, flags, eps,
                               out, topk_idx, offsets, perm_src,
                               reinterpret_cast<float *>(base + w.logits),
                               reinterpret_cast<unsigned int *>(base + w.sync), st);
    } else {
      e = launch_combine(L, y_perm, ys, inv_pos, topk_w, T, flags, eps, out, st);
      if (e == hipSuccess && i + 1 < n)
        e = run_route_permute(*layers[i + 1], out, T, topk_idx, topk_w, offsets, perm_src,
                              inv_pos, nullptr, base, w, st);
    }
    in = out;
  }
  return hip_status(e);
}

// Every argument of a whole-layer call but the workspace.
static moe_status check_layer_call(const moe_layer *L, const uint16_t *x, int32_t T,
                                   const int32_t *topk_idx, const float *topk_w,
                                   const int32_t *offsets, const int32_t *perm_src,
                                   const int32_t *inv_pos, const uint16_t *x_perm,
                                   const uint16_t *y_perm, const uint16_t *y_shared,
                                   uint32_t flags, float eps, const uint16_t *out) {
  moe_status s;
  if ((s = check_route_args(L, x, topk_idx, topk_w)) != MOE_OK) return s;
  if ((s = check_permute_args(x, topk_idx, offsets, perm_src, inv_pos, x_perm)) != MOE_OK)
    return s;
  if ((s = check_ffn_args(L, T, x, x_perm, perm_src, offsets, y_perm, y_shared)) != MOE_OK)
    return s;
  const uint16_t *ys = L->shared_ffn > 0 ? y_shared : nullptr;
  return check_combine_args(y_perm, ys, inv_pos, topk_w, flags, eps, out);
}

// Fixed scratch of moe_layer_forward_noalloc: a __device__ array exists once
// on every GPU the library is loaded on.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): it
// looks up each device's address once, with that device current, and passes
// that address.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static char *g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// The current device's scratch address.  On the first call for a device:
// look it up and zero-fill the counter block at its start on `st` (a fill
// kernel; later calls leave the block at zero).
static moe_status device_scratch(hipStream_t st, char **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u)) return MOE_EHIP;
    hipLaunchKernelGGL(zero_words_kernel, dim3(kWsSyncBytes / 16 / 256), dim3(256), 0, st,
                       static_cast<u32x4 *>(ptr), (size_t)(kWsSyncBytes / 16));
    if ((e = hipGetLastError()) != hipSuccess) return hip_status(e);
    g_scratch_ptr[dev] = static_cast<char *>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_size(const moe_layer *layer, int32_t max_tokens) {
  if (check_layer(layer) != MOE_OK || max_tokens < 0) return 0;
  return ws_layout(*layer, max_tokens).total;
}

moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  if (ws_bytes < kWsSyncBytes) return MOE_EWORKSPACE;
  if (!ok_ptr(ws)) return MOE_EINVAL;
  clear_stale_hip_error();
  hipLaunchKernelGGL(zero_words_kernel, dim3(kWsSyncBytes / 16 / 256), dim3(256), 0,
                     (hipStream_t)stream, static_cast<u32x4 *>(ws), (size_t)(kWsSyncBytes / 16));
  return hip_status(hipGetLastError());
}

moe_status moe_route(const moe_layer *L, const uint16_t *x, int32_t T, int32_t *topk_idx,
                     float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  moe_status s;
  if ((s = check_layer(L)) != MOE_OK) return s;
  if ((s = check_tokens(L, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_route_args(L, x, topk_idx, topk_w)) != MOE_OK) return s;
  if ((s = check_ws(L, T, ws, ws_bytes)) != MOE_OK) return s;
  const WsLayout w = ws_layout(*L, T);
  float *logits = reinterpret_cast<float *>(static_cast<char *>(ws) + w.logits);
  clear_stale_hip_error();
  return hip_status(launch_route(*L, x, T, topk_idx, topk_w, logits, (hipStream_t)stream));
}

moe_status moe_permute(const moe_layer *L, const uint16_t *x, const int32_t *topk_idx, int32_t T,
                       int32_t *offsets, int32_t *perm_src, int32_t *inv_pos, uint16_t *x_perm,
                       void *ws, size_t ws_bytes, void *stream) {
  moe_status s;
  if ((s = check_layer(L)) != MOE_OK) return s;
  if ((s = check_tokens(L, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_permute_args(x, topk_idx, offsets, perm_src, inv_pos, x_perm)) != MOE_OK)
    return s;
  if ((s = check_ws(L, T, ws, ws_bytes)) != MOE_OK) return s;
  const WsLayout w = ws_layout(*L, T);
  char *base = static_cast<char *>(ws);
  clear_stale_hip_error();
  return hip_status(launch_permute(*L, x, topk_idx, T, offsets, perm_src, inv_pos, x_perm,
                                   reinterpret_cast<int32_t *>(base + w.counts),
                                   reinterpret_cast<int32_t *>(base + w.bases),
                                   (hipStream_t)stream));
}

moe_status moe_route_permute(const moe_layer *L, const uint16_t *x, int32_t T, int32_t *topk_idx,
                             float *topk_w, int32_t *offsets, int32_t *perm_src, int32_t *inv_pos,
                             uint16_t *x_perm, void *ws, size_t ws_bytes, void *stream) {
  moe_status s;
  if ((s = check_layer(L)) != MOE_OK) return s;
  if ((s = check_tokens(L, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_route_args(L, x, topk_idx, topk_w)) != MOE_OK) return s;
  if ((s = check_permute_args(x, topk_idx, offsets, perm_src, inv_pos, x_perm)) != MOE_OK)
    return s;
  if ((s = check_ws(L, T, ws, ws_bytes)) != MOE_OK) return s;
  const WsLayout w = ws_layout(*L, T);
  clear_stale_hip_error();
  return hip_status(run_route_permute(*L, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos,
                                      x_perm, static_cast<char *>(ws), w, (hipStream_t)stream));
}

moe_status moe_w4_grouped_ffn(const moe_layer *L, const uint16_t *x, const uint16_t *x_perm,
                              const int32_t *perm_src, const int32_t *offsets, int32_t T,
                              uint16_t *y_perm, uint16_t *y_shared, void *ws, size_t ws_bytes,
                              void *stream) {
  moe_status s;
  if ((s = check_layer(L)) != MOE_OK) return s;
  if ((s = check_tokens(L, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_ffn_args(L, T, x, x_perm, perm_src, offsets, y_perm, y_shared)) != MOE_OK)
    return s;
  if ((s = check_ws(L, T, ws, ws_bytes)) != MOE_OK) return s;
  const WsLayout w = ws_layout(*L, T);
  char *base = static_cast<char *>(ws);
  clear_stale_hip_error();
  return hip_status(launch_ffn(*L, x, x_perm, perm_src, offsets, T, y_perm,
                               L->shared_ffn > 0 ? y_shared : nullptr,
                               reinterpret_cast<uint16_t *>(base + w.h),
                               reinterpret_cast<uint16_t *>(base + w.h_shared),
                               reinterpret_cast<float *>(base + w.split), ffn_tickets(base, w),
                               (hipStream_t)stream));
}

moe_status moe_unpermute_combine(const moe_layer *L, const uint16_t *y_perm,
                                 const uint16_t *y_shared, const int32_t *inv_pos,
                                 const float *topk_w, int32_t T, uint32_t flags, float eps,
                                 uint16_t *out, void *stream) {
  moe_status s;
  if ((s = check_layer(L)) != MOE_OK) return s;
  if ((s = check_tokens(L, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_combine_args(y_perm, y_shared, inv_pos, topk_w, flags, eps, out)) != MOE_OK)
    return s;
  clear_stale_hip_error();
  return hip_status(launch_combine(*L, y_perm, y_shared, inv_pos, topk_w, T, flags, eps, out,
                                   (hipStream_t)stream));
}

moe_status moe_layer_forward(const moe_layer *L, const uint16_t *x, int32_t T, int32_t *topk_idx,
                             float *topk_w, int32_t *offsets, int32_t *perm_src, int32_t *inv_pos,
                             uint16_t *x_perm, uint16_t *y_perm, uint16_t *y_shared,
                             uint32_t flags, float eps, uint16_t *out, void *ws, size_t ws_bytes,
                             void *stream) {
  moe_status s;
  if ((s = check_layer(L)) != MOE_OK) return s;
  if ((s = check_tokens(L, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_layer_call(L, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm,
                            y_perm, y_shared, flags, eps, out)) != MOE_OK)
    return s;
  if ((s = check_ws(L, T, ws, ws_bytes)) != MOE_OK) return s;
  clear_stale_hip_error();
  return run_layer(*L, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm, y_perm,
                   L->shared_ffn > 0 ? y_shared : nullptr, flags, eps, out,
                   static_cast<char *>(ws), (hipStream_t)stream);
}

moe_status moe_decode_stack_forward(const moe_layer *const *layers, int32_t n_layers,
                                    const uint16_t *x, int32_t T, int32_t *topk_idx,
                                    float *topk_w, int32_t *offsets, int32_t *perm_src,
                                    int32_t *inv_pos, uint16_t *y_perm, uint16_t *y_shared,
                                    uint32_t flags, float eps, uint16_t *acts, void *ws,
                                    size_t ws_bytes, void *stream) {
  if (!layers || n_layers < 1) return MOE_EINVAL;
  moe_status s;
  const moe_layer *L0 = layers[0];
  for (int32_t i = 0; i < n_layers; ++i) {
    const moe_layer *L = layers[i];
    if ((s = check_layer(L)) != MOE_OK) return s;
    if (L->num_experts != L0->num_experts || L->hidden != L0->hidden || L->ffn != L0->ffn ||
        L->top_k != L0->top_k || L->shared_ffn != L0->shared_ffn)
      return MOE_EUNSUPPORTED;
  }
  if ((s = check_tokens(L0, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  for (int32_t i = 0; i < n_layers; ++i)
    if ((s = check_layer_call(layers[i], x, T, topk_idx, topk_w, offsets, perm_src, inv_pos,
                              nullptr, y_perm, y_shared, flags, eps, acts)) != MOE_OK)
      return s;
  if ((s = check_ws(L0, T, ws, ws_bytes)) != MOE_OK) return s;
  clear_stale_hip_error();
  return run_stack(layers, n_layers, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, y_perm,
                   L0->shared_ffn > 0 ? y_shared : nullptr, flags, eps, acts,
                   static_cast<char *>(ws), (hipStream_t)stream);
}

moe_status moe_layer_forward_noalloc(const moe_layer *L, const uint16_t *x, int32_t T,
                                     int32_t *topk_idx, float *topk_w, int32_t *offsets,
                                     int32_t *perm_src, int32_t *inv_pos, uint16_t *x_perm,
                                     uint16_t *y_perm, uint16_t *y_shared, uint32_t flags,
                                     float eps, uint16_t *out, void *stream) {
  moe_status s;
  if ((s = check_layer(L)) != MOE_OK) return s;
  if ((s = check_tokens(L, T)) != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if ((s = check_layer_call(L, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm,
                            y_perm, y_shared, flags, eps, out)) != MOE_OK)
    return s;
  if (ws_layout(*L, T).total > kScratchBytes) return MOE_EWORKSPACE;
  const hipStream_t st = (hipStream_t)stream;
  clear_stale_hip_error();
  char *base = nullptr;
  if ((s = device_scratch(st, &base)) != MOE_OK) return s;
  return run_layer(*L, x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm, y_perm,
                   L->shared_ffn > 0 ? y_shared : nullptr, flags, eps, out, base, st);
}

moe_status moe_w4_dequant(const uint8_t *q, const uint16_t *s, int64_t rows, int64_t cols,
                          int32_t group_size, float *out, void *stream) {
  if (rows < 0 || cols < 0) return MOE_EINVAL;
  if (!supported_group_size(group_size)) return MOE_EUNSUPPORTED;
  if (cols % 128 || cols % group_size || rows % 16) return MOE_EUNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if ((rows * (cols / 8) + 255) / 256 > 0x7fffffffLL) return MOE_EUNSUPPORTED;
  if (!ok_ptr(q) || !ok_ptr(s) || !ok_ptr(out)) return MOE_EINVAL;
  clear_stale_hip_error();
  return hip_status(launch_dequant(q, s, rows, cols, group_size, out, (hipStream_t)stream));
}

moe_status moe_w4_quantize(const uint16_t *w, int64_t rows, int64_t cols, int32_t group_size,
                           uint8_t *q, uint16_t *s, void *stream) {
  if (rows < 0 || cols < 0) return MOE_EINVAL;
  if (!supported_group_size(group_size)) return MOE_EUNSUPPORTED;
  if (cols % 128 || cols % group_size || rows % 16) return MOE_EUNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if ((rows * (cols / 8) + 255) / 256 > 0x7fffffffLL) return MOE_EUNSUPPORTED;
  if (!ok_ptr(w) || !ok_ptr(q) || !ok_ptr(s)) return MOE_EINVAL;
  clear_stale_hip_error();
  return hip_status(launch_quantize(w, rows, cols, group_size, q, s, (hipStream_t)stream));
}

moe_status moe_w4_pack(const uint8_t *q_rowmajor, const uint16_t *s_rowmajor, int64_t rows,
                       int64_t cols, int32_t group_size, uint8_t *q, uint16_t *s, void *stream) {
  if (rows < 0 || cols < 0) return MOE_EINVAL;
  if (!supported_group_size(group_size)) return MOE_EUNSUPPORTED;
  if (cols % 128 || cols % group_size || rows % 16) return MOE_EUNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if ((rows * (cols / 8) + 255) / 256 > 0x7fffffffLL) return MOE_EUNSUPPORTED;
  if (!ok_ptr(q_rowmajor) || !ok_ptr(s_rowmajor) || !ok_ptr(q) || !ok_ptr(s)) return MOE_EINVAL;
  clear_stale_hip_error();
  return hip_status(launch_pack(q_rowmajor, s_rowmajor, rows, cols, group_size, q, s,
                                (hipStream_t)stream));
}

moe_status moe_w8_quantize(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *q, uint16_t *s,
                           void *stream) {
  if (rows < 0 || cols < 0) return MOE_EINVAL;
  if (cols % 128 || rows % 16) return MOE_EUNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if ((rows * (cols / 8) + 255) / 256 > 0x7fffffffLL) return MOE_EUNSUPPORTED;
  if (!ok_ptr(w) || !ok_ptr(q) || !ok_ptr(s)) return MOE_EINVAL;
  clear_stale_hip_error();
  return hip_status(launch_quantize8(w, rows, cols, q, s, (hipStream_t)stream));
}

const char *moe_last_hip_error(void) {
  return g_last_hip_error == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip_error);
}

const char *moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null or misaligned pointer, negative size, bad flag)";
    case MOE_EUNSUPPORTED: return "unsupported shape (group size 64/128/256, hidden/ffn multiple "
                                  "of 128 and of the group size, top_k, expert count)";
    case MOE_EWORKSPACE: return "workspace smaller than moe_workspace_size()";
    case MOE_EHIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}

}  // extern "C"
