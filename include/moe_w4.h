/*
 * moe_w4.h -- C ABI of the MI355X (gfx950) sparse-MoE expert layer with
 * 4-bit group-quantized experts.
 *
 * One MoE layer forward is four calls, in this order, on one stream:
 *
 *   moe_route              router logits + softmax + top-k
 *   moe_permute            per-expert token segments (histogram, scan, scatter)
 *   moe_w4_grouped_ffn     SwiGLU FFN of every routed expert over its segment,
 *                          int4 weights dequantized inside the kernel, plus the
 *                          always-on shared expert (fp16, or 8-bit)
 *   moe_unpermute_combine  weighted sum of each token's k expert outputs plus
 *                          the shared expert's output (optional RMS norm)
 *
 * moe_route_permute does the first two in one call (one launch for small
 * batches) and moe_layer_forward all four; moe_decode_stack_forward runs a
 * decode step through a stack of layers.  moe_w4_quantize and
 * moe_w8_quantize write the weight formats below from fp16 matrices;
 * moe_w4_pack writes the int4 format from codes that are already quantized
 * and stored plainly (row-major, two's-complement nibbles).
 *
 * Sources: symmetric int4 group quantization with 128 weights per group along
 * in_features, scale = max|w| / 7, codes clamped to [-8, 7]: lpnh.cn/news/
 * 2730718 §2.1 (quantization strategy, pseudo-code).  Softmax over the expert
 * logits and a descending partial sort for the top k: zwxr.cn/news/276292
 * §3.2 (routing engine); softmax and top-k fused in one kernel: lpnh.cn/news/
 * 2730718 §2.3.  Tokens that chose the same expert grouped for one grouped
 * GEMM launch: xdnf.cn/news/329730 §3.2.  Gate / up / down expert matrices and
 * "8 routed + 1 shared" experts per token: haowenji.com/articles/
 * x-2109226022155796480 §01.
 *
 * Conventions for every call
 * --------------------------
 *  - Every pointer argument is a DEVICE pointer unless marked "host".  fp16
 *    data is passed as uint16_t bit patterns (IEEE binary16).
 *  - Every device pointer must be 16-byte aligned.
 *  - The caller allocates and owns every buffer, including the workspace;
 *    the library never allocates, frees or keeps a pointer after a call
 *    returns.  Calls are asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream), never synchronize the host and never read device memory
 *    from the host, so a whole layer can be captured into a HIP graph.
 *  - Outputs are overwritten, never accumulated.  No floating-point atomics
 *    are used: the same inputs give bitwise identical outputs.
 *  - Arguments are checked on the host before anything is launched; a failed
 *    check launches nothing and returns a negative moe_status.  T = 0 returns
 *    MOE_OK and launches nothing.
 *  - Two calls that share a workspace must not run concurrently.  Prepare a
 *    workspace once before its first use with moe_workspace_init (or zero-fill
 *    its first 16384 bytes): they hold synchronization counters that every
 *    call leaves at zero.  A workspace whose counter is not zero makes
 *    moe_route_permute and moe_layer_forward write no routing (no error can be
 *    reported without reading device memory on the host).
 *
 * Packed int4 weight format (this library's choice; the page stores int8
 * codes).  A matrix [out, in] with group size gs (out a multiple of 16, in a
 * multiple of 128 and of gs) is stored as out*in/2 bytes of codes plus
 * out*in/gs fp16 scales.  A code q in
 * [-8, 7] is the nibble u = q + 8.  Eight consecutive columns 8w..8w+7 of a
 * row form one little-endian 32-bit word whose nibble p (bits 4p..4p+3) holds
 * column 8w + {0,2,4,6,1,3,5,7}[p]; four words (32 columns) form a 16-byte
 * chunk.  Rows are stored in tiles of 16, the 16 rows' chunks side by side,
 * so the 16 rows x 128 columns of one block are 1 KB contiguous (the weight
 * layout is reordered for contiguous access, as dpshk.com/news/6309482 §3.2
 * recommends):
 *     byte(row n, chunk c, b) = (n/16)*16*(in/2) + c*256 + (n%16)*16 + b
 *     scale(row n, group g)   = (n/16)*16*(in/gs) + g*16 + n%16
 * The dequantized weight is W[n][c] = q[n][c] * scale[n][c / gs].  The code
 * layout does not depend on gs.  gs is 128 (lpnh.cn/news/2730718 §2.1), or
 * 64 or 256, the sizes that page compares it with (§2.1) and suggests trying
 * when quality drops (64, §4.1).
 */
#ifndef MOE_W4_H
#define MOE_W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* null / misaligned pointer, negative size        */
    MOE_EUNSUPPORTED = -2,  /* shape outside what the kernels implement        */
    MOE_EWORKSPACE = -3,    /* ws_bytes smaller than moe_workspace_size()      */
    MOE_EHIP = -4           /* the HIP runtime reported an error at launch     */
} moe_status;

/* One MoE layer.  A HOST struct holding DEVICE pointers.
 *
 *  num_experts  E, 1..1024
 *  hidden       H, multiple of 128, <= 65536
 *  ffn          F (per routed expert), multiple of 128
 *  top_k        k, 1..min(E, 32)
 *  group_size   gs: 64, 128 or 256; hidden and ffn must be multiples of it
 *  router_w     fp16 [E, H]
 *  router_b     fp32 [E], or NULL for no bias (added to the logits before the
 *               softmax, so it also changes the combine weights)
 *  gate_q, up_q packed int4, E matrices [F, H] back to back (E*F*H/2 bytes);
 *               gate_s, up_s their fp16 scales (E*F*H/gs)
 *  down_q       packed int4, E matrices [H, F] (E*H*F/2 bytes); down_s scales
 *  shared_ffn   Fs of the always-on shared expert, multiple of 128, or 0
 *  shared_bits  16 (or 0): the shared expert's weights are fp16,
 *                 shared_gate, shared_up  fp16 [Fs, H];  shared_down  fp16 [H, Fs]
 *               8: they are 8-bit with 128-weight groups, as
 *                 xdnf.cn/news/329730 §3.1 keeps the shared FFN (the 8-bit
 *                 format below), shared_gate_q / shared_up_q [Fs, H] and
 *                 shared_down_q [H, Fs] codes with their fp16 scales
 *                 shared_gate_s / shared_up_s [Fs, H/128], shared_down_s
 *                 [H, Fs/128]; the fp16 pointers are then unused
 *
 * 8-bit format (shared expert): a matrix [out, in] (out a multiple of 16, in
 * of 128) is out*in bytes of codes plus out*in/128 fp16 scales; the code q in
 * [-128, 127] is the byte q + 128; rows in tiles of 16 with each 16-column
 * chunk of the 16 rows side by side:
 *     byte(row n, col c)    = (n/16)*16*in + (c/16)*256 + (n%16)*16 + c%16
 *     scale(row n, group g) = (n/16)*16*(in/128) + g*16 + n%16
 * W[n][c] = q[n][c] * scale[n][c / 128].
 */
typedef struct moe_layer {
    int32_t num_experts;
    int32_t hidden;
    int32_t ffn;
    int32_t top_k;
    int32_t group_size;
    int32_t shared_ffn;
    const uint16_t *router_w;
    const float *router_b;
    const uint8_t *gate_q;
    const uint16_t *gate_s;
    const uint8_t *up_q;
    const uint16_t *up_s;
    const uint8_t *down_q;
    const uint16_t *down_s;
    const uint16_t *shared_gate;
    const uint16_t *shared_up;
    const uint16_t *shared_down;
    int32_t shared_bits;
    const uint8_t *shared_gate_q;
    const uint16_t *shared_gate_s;
    const uint8_t *shared_up_q;
    const uint16_t *shared_up_s;
    const uint8_t *shared_down_q;
    const uint16_t *shared_down_s;
} moe_layer;

/* Bytes of workspace that every call below needs for up to `max_tokens`
 * tokens of `layer` (one workspace serves all four calls).  Returns 0 when
 * the layer description is invalid.  `layer` is a host pointer. */
size_t moe_workspace_size(const moe_layer *layer, int32_t max_tokens);

/* Prepare a workspace for its first use: zero-fills its first 16384 bytes (the
 * counter block) with a kernel on `stream` (no memset, so the call may also be
 * captured into a graph).  ws_bytes below 16384: MOE_EWORKSPACE; ws NULL or
 * misaligned: MOE_EINVAL.  Calls after the first leave the block at zero, so
 * one init per workspace is enough (again after a run that was aborted). */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Router: l[t][e] = sum_h x[t][h] * router_w[e][h] + router_b[e] (fp32
 * accumulation), p = softmax over e (fp32, max subtracted), then the k largest
 * logits in descending order, ties to the lower expert index.
 * Defined by zwxr.cn/news/276292 §3.2 (routing engine: softmax over the
 * expert logits, descending partial sort for the first k) and lpnh.cn/news/
 * 2730718 §2.3 (softmax and top-k fused in one kernel); the tie order is this
 * library's (the page's partial sort leaves ties open).
 *   x         fp16 [T, H]
 *   topk_idx  int32 [T, k]  out: chosen experts, best first
 *   topk_w    fp32  [T, k]  out: p of the chosen experts (not renormalised)
 * Logits that are NaN rank below every number; the k indices are always
 * distinct and in [0, E). */
moe_status moe_route(const moe_layer *layer, const uint16_t *x, int32_t T,
                     int32_t *topk_idx, float *topk_w,
                     void *ws, size_t ws_bytes, void *stream);

/* Permutation of the T*k (token, slot) pairs into per-expert segments.
 * Flat index f = t*k + j; segment e holds the f with topk_idx[f] = e in
 * increasing f.  The tokens that chose an expert are gathered so that each
 * expert runs once over all of them (xdnf.cn/news/329730 §3.2, grouped GEMM
 * over the selected experts); the stable order inside a segment is this
 * library's.
 *   x         fp16 [T, H] (read only when x_perm is not NULL)
 *   topk_idx  int32 [T, k], each in [0, E)
 *   offsets   int32 [E+1] out: segment e is rows offsets[e]..offsets[e+1]-1
 *   perm_src  int32 [T*k] out: flat index f of permuted row r
 *   inv_pos   int32 [T*k] out: permuted row of flat index f
 *   x_perm    fp16 [T*k, H] out: x_perm[r] = x[perm_src[r] / k] (bit copy),
 *             or NULL to skip the copy (moe_w4_grouped_ffn can read the rows
 *             of x through perm_src)
 * Indices outside [0, E) are clamped into range on the device so no access
 * leaves the buffers; such input is a caller error and gives unspecified
 * (but in-bounds) segments. */
moe_status moe_permute(const moe_layer *layer, const uint16_t *x,
                       const int32_t *topk_idx, int32_t T,
                       int32_t *offsets, int32_t *perm_src, int32_t *inv_pos,
                       uint16_t *x_perm, void *ws, size_t ws_bytes, void *stream);

/* moe_route followed by moe_permute, same arguments and outputs as the two
 * calls.  For T <= 64 and T*E <= 8192 both run in one launch: the last router block to finish
 * (a device-wide counter in the workspace) runs the softmax, top-k and the
 * permutation, so the workspace must be zero-filled before its first use
 * (every call leaves that counter at zero again). */
moe_status moe_route_permute(const moe_layer *layer, const uint16_t *x, int32_t T,
                             int32_t *topk_idx, float *topk_w, int32_t *offsets,
                             int32_t *perm_src, int32_t *inv_pos, uint16_t *x_perm,
                             void *ws, size_t ws_bytes, void *stream);

/* Grouped SwiGLU FFN over the routed segments and the shared expert: one
 * grouped GEMM over the selected experts' segments (xdnf.cn/news/329730 §3.2)
 * with the int4 weights of lpnh.cn/news/2730718 §2.1 dequantized inside the
 * kernel, gate / up / down matrices per expert (haowenji.com/articles/
 * x-2109226022155796480 §01).
 * For each expert e and each row r of its segment, with a = x_perm[r], or
 * a = x[perm_src[r] / k] when x_perm is NULL:
 *   g = deq(gate_e) a,  u = deq(up_e) a          (fp32 accumulation)
 *   h = silu(g) * u  with silu(z) = z / (1 + exp(-z)), stored as fp16
 *   y_perm[r] = deq(down_e) h                    (fp32 accumulation)
 * and, when the layer has a shared expert, the same with its fp16 weights for
 * every token of x, into y_shared.
 *   x         fp16 [T, H]   (needed when x_perm is NULL or shared_ffn > 0)
 *   x_perm    fp16 [T*k, H] or NULL;  perm_src int32 [T*k] (needed when
 *             x_perm is NULL; then T*H*2 must be below 2^31, else
 *             MOE_EUNSUPPORTED);  offsets int32 [E+1] as written by moe_permute
 *             (offsets[0] = 0, non-decreasing, offsets[E] = T*k)
 *   y_perm    fp16 [T*k, H] out
 *   y_shared  fp16 [T, H] out, or NULL when shared_ffn = 0
 * Kernel choice (results meet the same definition either way): the matrix-
 * core prefill kernels run the routed experts when T*k >= 32*E (segments of
 * 32 rows or more on average), hidden % 256 == 0 and T*k*H*2, T*k*F*2 and
 * F*H/2 are all below 2^31 (they address activations and one expert's
 * weights with 32-bit offsets); otherwise the decode kernels do, which are
 * correct at any size but read each expert's weights once per 16 rows of its
 * segment, so a large batch outside those limits runs far slower.  For up to
 * 16 tokens the decode kernels may split the in_features of each product over
 * several blocks whose fp32 partial sums are added in a fixed order (the
 * workspace holds them; outputs stay bitwise reproducible). */
moe_status moe_w4_grouped_ffn(const moe_layer *layer, const uint16_t *x,
                              const uint16_t *x_perm, const int32_t *perm_src,
                              const int32_t *offsets, int32_t T,
                              uint16_t *y_perm, uint16_t *y_shared,
                              void *ws, size_t ws_bytes, void *stream);

#define MOE_RMSNORM 1u
#define MOE_RENORM 2u

/* Combine: out[t] = y_shared[t] + sum_j topk_w[t][j] * y_perm[inv_pos[t*k+j]]
 * in fp32 (y_shared may be NULL: then that term is 0): the k routed experts'
 * outputs weighted by their routing probabilities plus the always-on shared
 * expert with weight 1 (haowenji.com/articles/x-2109226022155796480 §01,
 * "8 routed + 1 shared" experts per token).  With flags &
 * MOE_RENORM each topk_w[t][j] is first divided by the sum of the token's k
 * weights (the chosen experts' probabilities rescaled to sum to 1; an option
 * beyond the pages, whose routing keeps the plain softmax probabilities).
 * With flags & MOE_RMSNORM the row is then divided by
 * sqrt(mean(row^2) + eps) (no gain, no residual), as between stacked layers.
 * Stored as fp16.
 *   out  fp16 [T, H] out.  inv_pos entries must lie in [0, T*k) (clamped on
 *        the device otherwise). */
moe_status moe_unpermute_combine(const moe_layer *layer, const uint16_t *y_perm,
                                 const uint16_t *y_shared, const int32_t *inv_pos,
                                 const float *topk_w, int32_t T, uint32_t flags,
                                 float eps, uint16_t *out, void *stream);

/* One whole layer forward in one call: moe_route_permute,
 * moe_w4_grouped_ffn and moe_unpermute_combine run in that order on `stream`
 * with these arguments, and every output is bitwise what those three calls
 * give (fewer host calls per layer; per-launch overhead is the concern of
 * xdnf.cn/news/329730 §3.2, grouped GEMM and CUDA Graph).
 *   x, T, topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm  as in
 *        moe_route_permute (x_perm may be NULL; then T*H*2 must be below
 *        2^31, else MOE_EUNSUPPORTED)
 *   y_perm, y_shared  as in moe_w4_grouped_ffn (y_shared NULL when
 *        shared_ffn = 0; ignored then)
 *   flags, eps, out   as in moe_unpermute_combine, with y_shared as its
 *        shared term
 * All arguments are checked before the first launch. */
moe_status moe_layer_forward(const moe_layer *layer, const uint16_t *x, int32_t T,
                             int32_t *topk_idx, float *topk_w, int32_t *offsets,
                             int32_t *perm_src, int32_t *inv_pos, uint16_t *x_perm,
                             uint16_t *y_perm, uint16_t *y_shared, uint32_t flags,
                             float eps, uint16_t *out, void *ws, size_t ws_bytes,
                             void *stream);

/* A decode step through n_layers stacked layers, the output of layer i being
 * the input of layer i + 1 (haowenji.com/articles/x-2109226022155796480 §01:
 * a decode step runs the token through 42 MoE layers).  Computes
 *     acts[0] = layer_0(x),  acts[i] = layer_i(acts[i-1]),
 * each layer_i being moe_layer_forward of layers[i] with x_perm NULL and the
 * given flags and eps (MOE_RMSNORM between stacked layers).
 *   layers    HOST array of n_layers (>= 1) host pointers; every layer has
 *             the same num_experts, hidden, ffn, top_k and shared_ffn
 *             (MOE_EUNSUPPORTED otherwise); group sizes and shared_bits may
 *             differ
 *   x         fp16 [T, H], the input of layer 0; T*H*2 below 2^31
 *   acts      fp16 [n_layers, T, H] out: every layer's output, the last one
 *             being the step's output
 *   topk_idx, topk_w, offsets, perm_src, inv_pos, y_perm, y_shared
 *             as in moe_layer_forward; reused by every layer, they hold the
 *             last layer's values when the call returns
 *   flags, eps, ws, ws_bytes, stream  as in moe_layer_forward; the workspace
 *             is moe_workspace_size(layers[0], T) bytes
 * Launches: for T <= 32 tokens and hidden <= 8192 the combine of layer i and
 * the router, top-k and permutation of layer i + 1 run in one launch (one
 * block per token and tile of experts forms the token's combined row, the
 * last block of each token runs its top-k, the last of those the
 * permutation; the counter block of the workspace must start at zero, and
 * every call leaves it so).  The combined rows are bitwise those of
 * moe_unpermute_combine; the logits of layers 1 .. n-1 are fp32 dot products
 * summed in another order than moe_route's, so a token whose k-th and
 * (k+1)-th logits agree to the last bits may choose differently and the
 * combine weights may differ in the last bits.  Larger batches run each
 * layer as moe_layer_forward does, bitwise.  All arguments are checked
 * before the first launch. */
moe_status moe_decode_stack_forward(const moe_layer *const *layers, int32_t n_layers,
                                    const uint16_t *x, int32_t T, int32_t *topk_idx,
                                    float *topk_w, int32_t *offsets, int32_t *perm_src,
                                    int32_t *inv_pos, uint16_t *y_perm, uint16_t *y_shared,
                                    uint32_t flags, float eps, uint16_t *acts, void *ws,
                                    size_t ws_bytes, void *stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under graph capture without a memory pool, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and outputs without ws and
 * ws_bytes.  The workspace is instead a fixed array inside the library,
 * 16 MiB on every GPU the library is loaded on (held until the process
 * ends): a call whose moe_workspace_size(layer, T) exceeds 16 MiB returns
 * MOE_EWORKSPACE and launches nothing (decode batches fit: the 288-expert
 * hidden-4096 ffn-1536 top-8 layer with its shared expert up to 525 tokens,
 * the 16-expert hidden-12288 ffn-65536 top-4 layer up to 28; the 8192-token
 * prefill layer needs 262 MiB and does not).  The call allocates and frees nothing.  The first call on
 * a GPU looks up that GPU's copy of the array and zero-fills its counter
 * block on `stream`; `stream` must belong to the calling thread's current
 * device.  Every call on one GPU uses that GPU's one array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller. */
moe_status moe_layer_forward_noalloc(const moe_layer *layer, const uint16_t *x, int32_t T,
                                     int32_t *topk_idx, float *topk_w, int32_t *offsets,
                                     int32_t *perm_src, int32_t *inv_pos, uint16_t *x_perm,
                                     uint16_t *y_perm, uint16_t *y_shared, uint32_t flags,
                                     float eps, uint16_t *out, void *stream);

/* Test hook: out[n][c] = q[n][c] * s[n][c/gs] in fp32 (exact, row-major
 * [rows, cols]) for one matrix in the packed format above with group size
 * gs = group_size (64, 128 or 256); rows multiple of 16, cols multiple of 128
 * and of gs (MOE_EUNSUPPORTED otherwise). */
moe_status moe_w4_dequant(const uint8_t *q, const uint16_t *s, int64_t rows,
                          int64_t cols, int32_t group_size, float *out, void *stream);

/* Group quantization of an fp16 matrix w [rows, cols] in groups of
 * group_size columns (64, 128 or 256), lpnh.cn/news/2730718 §2.1 with every
 * step rounded to fp16 as on an fp16 model: s = RN16(max|w_group| / 7),
 * q = clamp(RNE(RN16(w / s)), -8, 7); an all-zero group gets s = 0, q = 0.
 * w is row-major; writes q and s in the packed format above.  rows multiple
 * of 16, cols multiple of 128 and of group_size. */
moe_status moe_w4_quantize(const uint16_t *w, int64_t rows, int64_t cols,
                           int32_t group_size, uint8_t *q, uint16_t *s, void *stream);

/* Codes that are already quantized, stored plainly, into the packed int4
 * format above (the page's quantizer returns int8 codes [out, in] with fp16
 * scales [out, in/group], lpnh.cn/news/2730718 §2.1; this call takes them
 * two codes per byte):
 *   q_rowmajor  [rows, cols/2] bytes, row-major; byte c/2 of a row holds
 *               column c (c even) in bits 0-3 and column c+1 in bits 4-7, each
 *               as a two's-complement nibble (codes -8..7)
 *   s_rowmajor  fp16 [rows, cols/group_size], row-major
 *   q, s        out: the packed format above (same byte and scale counts)
 * Bit-exact: codes and scales are moved, not recomputed.  rows multiple of 16,
 * cols multiple of 128 and of group_size (64, 128 or 256); MOE_EUNSUPPORTED
 * otherwise.  Inputs and outputs must not overlap. */
moe_status moe_w4_pack(const uint8_t *q_rowmajor, const uint16_t *s_rowmajor, int64_t rows,
                       int64_t cols, int32_t group_size, uint8_t *q, uint16_t *s, void *stream);

/* 8-bit group quantization of an fp16 matrix w [rows, cols] for the shared
 * expert (128-weight groups; xdnf.cn/news/329730 §3.1): the 4-bit steps of
 * moe_w4_quantize with 127 in place of 7 and codes clamped to [-128, 127]:
 * s = RN16(max|w_group| / 127), q = clamp(RNE(RN16(w / s)), -128, 127); an
 * all-zero group gets s = 0, q = 0.  Writes q and s in the 8-bit format
 * above.  rows multiple of 16, cols multiple of 128. */
moe_status moe_w8_quantize(const uint16_t *w, int64_t rows, int64_t cols,
                           uint8_t *q, uint16_t *s, void *stream);

/* Static description of a status code (host). */
const char *moe_status_str(moe_status status);

/* Host: the HIP runtime's message for the error behind the last MOE_EHIP
 * returned on the calling thread ("no HIP error" if there was none). */
const char *moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4_H */
