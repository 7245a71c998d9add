"""Float64 CPU oracle for the sparse MoE expert layer with W4 g128 experts.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test-suite, the smoke check
and the CPU-baseline leg of the benchmark may import this module.  It shares
no code with the HIP library: it is a plain, slow, obviously correct
restatement of what the layer computes, in float64, so that every GPU result
can be compared element by element against it.

Sources (web pages; cited by site, page section and the object on it):

  [P1] xdnf.cn/news/329730 "千亿MoE模型在RTX 3090上突破100 tok/s：全链路推理优化实战"
  [P2] lpnh.cn/news/2730718 (125B MoE on one RTX 3090, full-path tuning)
  [P3] zwxr.cn/news/276292 (Strata engine on RTX 3090 + Xeon E5-2699 v4)
  [P5] haowenji.com/articles/x-2109226022155796480
       "把 96.5GB 的 GLM-5.3-Flash 塞进单张 4090 48GB ..."

Each function names the passage it follows.  Readings taken where the pages
are silent or garbled are stated in the docstrings; the same list, with the
reasons, is kept in the design notes at the repository root.

Packed int4 storage (a format of this library, not of the pages, which keep
int8 codes).  Each code is stored as the unsigned nibble u = q + 8 (offset
binary, 0..15).  Eight consecutive columns 8w..8w+7 of a row form one 32-bit
little-endian word whose nibble p (bits 4p..4p+3) holds column
8w + (0, 2, 4, 6, 1, 3, 5, 7)[p]; four such words (32 columns) form a 16-byte
chunk.  A matrix [out, in] (out a multiple of 16, in a multiple of 128) is
stored tile by tile: 16 rows at a time, and inside a tile chunk by chunk with
the 16 rows' chunks side by side:

    byte offset(row n, chunk c, byte b) = (n // 16) * 16 * (in/2)
                                          + c * 256 + (n % 16) * 16 + b

so the 16 rows x 128 columns of one quantization group are 1 KB contiguous.
The fp16 scales [out, in/group] are stored the same way, 16 rows side by
side: offset(row n, group g) = (n // 16) * 16 * (in/group) + g * 16 + n % 16.
Both are kept as arrays of the logical shape [out, in/2] bytes and
[out, in/group] fp16 whose memory follows these offsets.

Group size: 128 everywhere unless a caller asks for 64 or 256, the two
neighbours [P2] §2.1 reports measuring (64: more scale metadata for no
speed; 256: quantization error starts to show) and the one [P2] §4.1
suggests trying when output quality drops (64).
"""
from __future__ import annotations

import numpy as np

GROUP = 128          # [P2] §2.1: 128 weights per group along in_features
QMAX = 7             # [P2] §2.1: 2**(bits-1) - 1 with bits = 4
QMIN, QHI = -8, 7    # [P2] §2.1: clamp range of the rounded codes


# ---------------------------------------------------------------------------
# fp16 rounding
# ---------------------------------------------------------------------------
def rn16(a) -> np.ndarray:
    """Round float64 values to the nearest fp16 (ties to even), back as float64.

    numpy converts float64 to float16 directly with round-to-nearest-even;
    the tests pin this against a brute-force nearest-neighbour search over
    every finite fp16 value.
    """
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# a0: symmetric group quantization  ([P2] §2.1 group-quantization pseudo-code;
#     applied offline to every module whose name contains "expert", [P2] §3.2)
# ---------------------------------------------------------------------------
def group_quantize(w16: np.ndarray, group: int = GROUP, bits: int = 4):
    """Quantize an fp16 weight [out, in] to int4 codes and fp16 group scales.

    [P2] §2.1: the weight is viewed as [out, in/group, group]; each group's
    scale is its largest magnitude divided by 2**(bits-1)-1 = 7; the codes are
    round(w / scale) clamped to [-8, 7].  The page runs this on a model loaded
    in fp16 ([P2] §3.2), so every operation rounds to fp16:

        s = RN16(max|w| / 7),   q = clamp(RNE(RN16(w / s)), -8, 7).

    bits = 8 gives the 8-bit weights [P1] §3.1 keeps for the shared FFN (with
    128-weight groups): the same steps with 2**(bits-1)-1 = 127 and the
    clamp range [-128, 127] (reading: the pages print only the 4-bit case).

    Each quotient is formed in float64 and then rounded once to fp16; since
    53 >= 2*11 + 2 this equals the correctly rounded fp16 quotient.  A group
    of zeros (0/0 on the page) gets s = 0 and q = 0 (reading: the page is
    silent).  in_features must be a multiple of the group size (reading: the
    page's reshape would drop a tail silently; here it is refused).

    Returns (q int8 [out, in], s float16 [out, in/group]).
    """
    w16 = np.asarray(w16)
    if w16.dtype != np.float16:
        raise TypeError("group_quantize expects fp16 weights")
    out_dim, in_dim = w16.shape
    if in_dim % group:
        raise ValueError("in_features must be a multiple of the group size")
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    qmax, qmin = 2 ** (bits - 1) - 1, -2 ** (bits - 1)
    w = w16.astype(np.float64).reshape(out_dim, in_dim // group, group)
    m = np.abs(w).max(axis=-1, keepdims=True)
    s = rn16(m / qmax)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = rn16(np.where(s > 0, w / np.where(s > 0, s, 1.0), 0.0))
    q = np.clip(np.rint(r), qmin, qmax)          # np.rint rounds half to even
    q = np.where(s > 0, q, 0.0)
    return (q.astype(np.int8).reshape(out_dim, in_dim),
            s.reshape(out_dim, in_dim // group).astype(np.float16))


# column offset (within a run of 8) held by the low / high nibble of byte b
_LO_COL = (0, 4, 1, 5)
_HI_COL = (2, 6, 3, 7)


def _rows_to_tiles(a: np.ndarray, unit: int) -> np.ndarray:
    """Row-major [out, n*unit] -> tile order: 16 rows side by side per unit."""
    out_dim, cols = a.shape
    t = a.reshape(out_dim // 16, 16, cols // unit, unit).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(t).reshape(out_dim, cols)


def _tiles_to_rows(a: np.ndarray, unit: int) -> np.ndarray:
    out_dim, cols = a.shape
    t = a.reshape(out_dim // 16, cols // unit, 16, unit).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(t).reshape(out_dim, cols)


def pack_w4(q: np.ndarray) -> np.ndarray:
    """int8 codes [out, in] in [-8, 7] -> stored bytes [out, in/2]."""
    q = np.asarray(q)
    if q.min(initial=0) < QMIN or q.max(initial=0) > QHI:
        raise ValueError("codes outside [-8, 7]")
    if q.shape[0] % 16 or q.shape[1] % GROUP:
        raise ValueError("out_features must be a multiple of 16, in_features of 128")
    u = (q.astype(np.int16) + 8).astype(np.uint8).reshape(q.shape[0], -1, 8)
    rows = np.empty((q.shape[0], q.shape[1] // 8, 4), dtype=np.uint8)
    for b in range(4):
        rows[:, :, b] = u[:, :, _LO_COL[b]] | (u[:, :, _HI_COL[b]] << 4)
    return _rows_to_tiles(rows.reshape(q.shape[0], q.shape[1] // 2), 16)


def unpack_w4(packed: np.ndarray) -> np.ndarray:
    """Stored bytes [out, in/2] -> int8 codes [out, in]."""
    p = _tiles_to_rows(np.asarray(packed, dtype=np.uint8), 16)
    p = p.reshape(p.shape[0], -1, 4)
    u = np.empty((p.shape[0], p.shape[1], 8), dtype=np.int8)
    for b in range(4):
        u[:, :, _LO_COL[b]] = (p[:, :, b] & 0x0F).astype(np.int8)
        u[:, :, _HI_COL[b]] = (p[:, :, b] >> 4).astype(np.int8)
    return (u - 8).reshape(p.shape[0], -1)


def unpack_plain_w4(b: np.ndarray) -> np.ndarray:
    """Plain int4 storage -> int8 codes [out, in].

    The plain layout is row-major [out, in/2] bytes; byte c/2 of a row holds
    column c (c even) in bits 0-3 and column c+1 in bits 4-7, each as a
    two's-complement nibble (a plain packing of the page's int8 codes,
    [P2] §2.1, two per byte; the library's own format is pack_w4's).
    """
    b = np.asarray(b, dtype=np.uint8)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    q = np.empty((b.shape[0], 2 * b.shape[1]), dtype=np.int8)
    q[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    q[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    return q


def pack_w8(q: np.ndarray) -> np.ndarray:
    """int8 codes [out, in] -> stored bytes [out, in]: the offset-binary byte
    q + 128, rows in tiles of 16 with each 16-column chunk of the 16 rows side
    by side, byte(n, c) = (n // 16) * 16 * in + (c // 16) * 256 + (n % 16) * 16
    + c % 16 (a format of this library for the 8-bit shared expert)."""
    q = np.asarray(q)
    if q.shape[0] % 16 or q.shape[1] % GROUP:
        raise ValueError("out_features must be a multiple of 16, in_features of 128")
    u = (q.astype(np.int16) + 128).astype(np.uint8)
    return _rows_to_tiles(u, 16)


def unpack_w8(packed: np.ndarray) -> np.ndarray:
    """Stored bytes [out, in] -> int8 codes [out, in]."""
    u = _tiles_to_rows(np.asarray(packed, dtype=np.uint8), 16)
    return (u.astype(np.int16) - 128).astype(np.int8)


def dequant_w8(packed: np.ndarray, s_stored: np.ndarray, group: int = GROUP) -> np.ndarray:
    """W[n, c] = q[n, c] * s[n, c // group] in float64 for a stored 8-bit matrix."""
    q = unpack_w8(packed).astype(np.float64)
    return q * np.repeat(unpack_scales(s_stored).astype(np.float64), group, axis=1)


def pack_scales(s: np.ndarray) -> np.ndarray:
    """fp16 scales [out, in/group] -> stored order (16 rows side by side)."""
    return _rows_to_tiles(np.asarray(s, dtype=np.float16), 1)


def unpack_scales(stored: np.ndarray) -> np.ndarray:
    return _tiles_to_rows(np.asarray(stored, dtype=np.float16), 1)


def dequant(packed: np.ndarray, s_stored: np.ndarray, group: int = GROUP) -> np.ndarray:
    """W[n, c] = q[n, c] * s[n, c // group] in float64, from the stored arrays
    (exact: an int4 code times an fp16 scale needs at most 4 + 11 bits)."""
    q = unpack_w4(packed).astype(np.float64)
    s64 = unpack_scales(s_stored).astype(np.float64)
    return q * np.repeat(s64, group, axis=1)


# ---------------------------------------------------------------------------
# a1 + a2: router logits, softmax, top-k
#   [P2] §2.3 (softmax and top-k fused in one kernel), [P3] §3.2 (softmax over
#   the expert logits, then a descending partial sort for the first k).
# ---------------------------------------------------------------------------
def router_logits(x16, wr16, bias=None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * Wr[e, h] + b[e]   (float64)."""
    l = np.asarray(x16, dtype=np.float64) @ np.asarray(wr16, dtype=np.float64).T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted first."""
    z = l - l.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def topk_order(l: np.ndarray, k: int) -> np.ndarray:
    """First k experts of each row ordered by (-logit, expert index).

    Reading: ties go to the lower expert index, both in selection and in the
    output order (the page's partial sort is unstable and leaves ties open).
    Top-k of the probabilities equals top-k of the logits: softmax is monotone.
    """
    T, E = l.shape
    eidx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((eidx, -l), axis=-1)   # last key primary: -logit, then index
    return order[:, :k].astype(np.int32)


def route(x16, wr16, bias, k: int, idx=None):
    """Returns (topk_idx int32 [T,k], topk_w float64 [T,k], logits float64 [T,E]).

    The combine weights are the softmax probabilities of the chosen experts,
    not renormalised over the k chosen (reading taken for every workload).

    idx: None, or a given selection int [T, k] (k distinct experts per row,
    each in [0, E)) used instead of the oracle's own top-k; the weights are
    then the probabilities of those experts.  This evaluates the layer on
    another implementation's choice at a reported near tie, where both
    selections are correct orderings of (numerically) equal logits.
    """
    l = router_logits(x16, wr16, bias)
    p = softmax(l)
    if idx is None:
        idx = topk_order(l, k)
    else:
        idx = np.asarray(idx)
        T, E = l.shape
        if idx.shape != (T, k):
            raise ValueError("given selection must be [T, k]")
        if idx.size and (idx.min() < 0 or idx.max() >= E):
            raise ValueError("given selection has an expert outside [0, E)")
        if any(len(set(row.tolist())) != k for row in idx):
            raise ValueError("given selection repeats an expert in a row")
        idx = idx.astype(np.int32)
    w = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return idx, w, l


# ---------------------------------------------------------------------------
# a3 + a4: token permutation by expert  ([P1] §3.2 and [P2] §2.3: tokens that
#   chose the same expert are gathered so that each expert runs one GEMM)
# ---------------------------------------------------------------------------
def permute(topk_idx: np.ndarray, num_experts: int):
    """Histogram, exclusive scan and stable scatter of the flat (token, slot) pairs.

    Flat index f = t*k + j.  Segment e holds the f with idx_flat[f] = e in
    increasing f (stable; reading taken so the permutation is unique).
    Returns (offsets int32 [E+1], perm_src int32 [T*k], inv_pos int32 [T*k]):
    perm_src[r] = f of the r-th permuted row, inv_pos[f] = r.
    """
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    cnt = np.bincount(flat, minlength=num_experts)
    off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    perm_src = np.argsort(flat, kind="stable").astype(np.int32)
    inv_pos = np.empty_like(perm_src)
    inv_pos[perm_src] = np.arange(flat.size, dtype=np.int32)
    return off, perm_src, inv_pos


def gather_rows(x16: np.ndarray, perm_src: np.ndarray, k: int) -> np.ndarray:
    """x_perm[r] = x[perm_src[r] // k] (a bitwise copy of fp16 rows)."""
    return np.asarray(x16)[np.asarray(perm_src, dtype=np.int64) // k]


# ---------------------------------------------------------------------------
# a5 + a6 + a7: SwiGLU expert FFN  ([P3] §4.3 and [P5] §01: each expert holds
#   gate / up / down matrices, Mixtral-style w1 / w3 / w2)
# ---------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """Y = (silu(X Wg^T) * (X Wu^T)) Wd^T, all float64.

    Wg, Wu are [F, H] (in_features = H), Wd is [H, F] (in_features = F).
    """
    X = np.asarray(X, dtype=np.float64)
    g = X @ np.asarray(Wg, dtype=np.float64).T
    u = X @ np.asarray(Wu, dtype=np.float64).T
    h = silu(g) * u
    return h @ np.asarray(Wd, dtype=np.float64).T


def expert_ffn_w4(X, gate_q, gate_s, up_q, up_s, down_q, down_s,
                  group: int = GROUP) -> np.ndarray:
    """One routed expert: dequantize its three int4 matrices (scales per
    `group` columns), then SwiGLU."""
    return swiglu_ffn(X, dequant(gate_q, gate_s, group), dequant(up_q, up_s, group),
                      dequant(down_q, down_s, group))


# ---------------------------------------------------------------------------
# a8: weighted combine + shared expert, and the RMS normalisation that links
#   stacked layers
# ---------------------------------------------------------------------------
def combine(y_perm, ys, inv_pos, topk_w, T: int, k: int, renorm: bool = False) -> np.ndarray:
    """out[t] = ys[t] + sum_j w[t, j] * y_perm[inv_pos[t*k + j]]  (float64).

    The shared expert enters with weight 1 and no gate ([P5] §01 "8 routed +
    1 shared"; reading: the shared expert is always on, unweighted).  With
    renorm, w[t, j] is replaced by w[t, j] / sum_j' w[t, j'] (an option beyond
    the pages, whose routing keeps the plain softmax probabilities).
    """
    y_perm = np.asarray(y_perm, dtype=np.float64)
    H = y_perm.shape[1] if y_perm.ndim == 2 and y_perm.shape[0] else (
        np.asarray(ys).shape[1] if ys is not None else 0)
    out = np.zeros((T, H)) if ys is None else np.asarray(ys, dtype=np.float64).copy()
    w = np.asarray(topk_w, dtype=np.float64).reshape(T, k)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    inv = np.asarray(inv_pos, dtype=np.int64).reshape(T, k)
    for j in range(k):
        out += w[:, j:j + 1] * y_perm[inv[:, j]]
    return out


def rmsnorm(y: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """y / sqrt(mean(y^2) + eps) per row; no learned gain, no residual.

    Reading: the stacked decode workload only says that a layer's output feeds
    the next layer after RMS normalisation.
    """
    y = np.asarray(y, dtype=np.float64)
    return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------
def moe_layer(x16, router_w16, router_b, experts, k: int, shared=None, expert_ffn=None,
              idx=None):
    """One MoE layer forward in float64, keeping every intermediate.

    experts: indexable by expert id, returning
             (gate_q, gate_s, up_q, up_s, down_q, down_s) for that expert
             (packed int4 bytes and fp16 scales).  Only the experts that
             receive tokens are fetched, so a lazy provider may regenerate
             them on demand.
    shared:  None or (Wg16 [Fs,H], Wu16 [Fs,H], Wd16 [H,Fs]) fp16.
    expert_ffn: the routed expert's FFN (default expert_ffn_w4; the C
             reference in oracle.cref evaluates the same definition for
             matrices too large to dequantize in numpy).
    idx:     None, or a given top-k selection [T, k] (see route): the layer
             evaluated on another implementation's experts at a reported
             near tie.
    """
    expert_ffn = expert_ffn_w4 if expert_ffn is None else expert_ffn
    x16 = np.asarray(x16)
    T = x16.shape[0]
    E = np.asarray(router_w16).shape[0]
    idx, w, logits = route(x16, router_w16, router_b, k, idx=idx)
    off, perm_src, inv_pos = permute(idx, E)
    x_perm = gather_rows(x16, perm_src, k)
    H = x16.shape[1]
    y_perm = np.zeros((T * k, H))
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            y_perm[a:b] = expert_ffn(x_perm[a:b], *experts[e])
    ys = swiglu_ffn(x16, *shared) if shared is not None else None
    out = combine(y_perm, ys, inv_pos, w, T, k)
    return dict(idx=idx, w=w, logits=logits, offsets=off, perm_src=perm_src,
                inv_pos=inv_pos, x_perm=x_perm, y_perm=y_perm, ys=ys, out=out)


def tie_excused(idx_other, logits: np.ndarray, gap: float = 1e-6):
    """Compare another implementation's ordered top-k lists with the oracle's.

    The workload contract: top-k indices are exact, and an index difference
    is reported rather than failed when it comes from a tie within 1e-6 of the
    logit gap.  Reading: position j of token t differs when the other list
    has expert a there and the oracle's list (order by -logit, then index)
    has expert b != a; that position is excused iff the float64 logits of a
    and b differ by at most `gap`.  A token is excused iff every differing
    position is; a token with a difference anywhere else is a failure.

    Returns (differs [T] bool, excused [T] bool); excused implies differs.
    """
    logits = np.asarray(logits, dtype=np.float64)
    other = np.asarray(idx_other, dtype=np.int64)
    T, k = other.shape
    ref = topk_order(logits, k).astype(np.int64)
    pos = other != ref
    differs = pos.any(axis=1)
    la = np.take_along_axis(logits, np.clip(other, 0, logits.shape[1] - 1), axis=1)
    lb = np.take_along_axis(logits, ref, axis=1)
    close = np.abs(la - lb) <= gap
    in_range = ((other >= 0) & (other < logits.shape[1])).all(axis=1)
    distinct = np.array([len(set(r.tolist())) == k for r in other], dtype=bool)
    excused = differs & in_range & distinct & (close | ~pos).all(axis=1)
    return differs, excused
