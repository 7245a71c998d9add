"""Full-size parity in the launch configuration the benchmark times
(moe_layer_forward for single layers: the one-launch router and permutation
for decode batches, the grouped FFN reading rows through perm_src, the
combine; moe_decode_stack_forward for the 42-layer decode step), against the
float64 oracle.

Expert weights are packed codes + scales drawn on the device with the law of
quantized N(0, sigma) weights (workloads.gen_torch); the oracle reads back the
experts it needs and evaluates them with the C reference products (decode) or
numpy (whole prefill segments).  Top-k indices must equal the oracle's except
at reported ties (oracle.tie_excused); outputs are then compared against the
oracle evaluated on the GPU's own selection, so no token is skipped.
"""

import numpy as np
import pytest
import torch

import oracle as O
from oracle import cref as C
from workloads import get_config
from workloads import gen as G
from workloads import gen_torch as GT

from gpu_util import gpu, require_gpu, tol_check, route_compare, shared_w8

pytestmark = gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _np(t):
    return t.detach().cpu().numpy()


def device_layer(cfg, layer_idx=0, w8=False):
    """w8: the shared expert stored in 8 bits (quantized by the oracle); the
    returned shared weights are then its float64 dequantized matrices."""
    from w4_group_quantized_amd import W4MoELayer
    dev = torch.device("cuda:0")
    mats = GT.layer_codes(cfg, layer_idx, dev)
    wr, b = G.router(cfg, layer_idx)
    shared = G.shared_expert(cfg, layer_idx)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    s8 = None
    if w8:
        stored, shared = shared_w8(shared)
        s8 = tuple((t(q), t(sc)) for q, sc in stored)
    layer = W4MoELayer(cfg.top_k, t(wr), t(b) if b is not None else None, mats["gate_q"],
                       mats["gate_s"], mats["up_q"], mats["up_s"], mats["down_q"], mats["down_s"],
                       shared=tuple(t(w) for w in shared) if shared is not None and not w8
                       else None, shared_w8=s8)
    return layer, mats, wr, b, shared


class DeviceExperts:
    """Lazy host copies of the experts the oracle needs."""

    def __init__(self, mats):
        self.mats, self.cache = mats, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = tuple(_np(self.mats[n][e]) for n in
                                  ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"))
        return self.cache[e]


def oracle_tokens(x64, wr, b, k, experts, shared, idx=None):
    """Float64 layer output for the given token rows (tokens are independent
    in an MoE layer), optionally on a given selection idx [n, k]."""
    idx, w, logits = O.route(x64, wr, b, k, idx=idx)
    out = O.swiglu_ffn(x64, *shared) if shared is not None else np.zeros((x64.shape[0], wr.shape[1]))
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        y = C.expert_ffn_w4_c(x64[rows], *experts[e])
        out[rows] += w[rows, slots][:, None] * y
    return out, idx, logits


def checked_tokens(x64, wr, b, k, experts, shared, idx_gpu):
    """The oracle's selection, then the GPU's checked against it under the
    tie rule; the output of the oracle on the GPU's selection."""
    logits = O.router_logits(x64, wr, b)
    route_compare(idx_gpu, logits, k)
    out, _, _ = oracle_tokens(x64, wr, b, k, experts, shared, idx=idx_gpu)
    return out


@pytest.mark.parametrize("name,n_sample", [("decode_fine", None), ("decode_coarse", None),
                                           ("prefill", 256), ("decode_fine512", None)])
def test_full_size_layer(name, n_sample):
    cfg = get_config(name)
    layer, mats, wr, b, shared = device_layer(cfg)
    T = cfg.tokens
    x = G.activations(cfg, batch=0)
    buf = layer.alloc(T)
    xd = torch.from_numpy(x).cuda()
    out = _np(layer.forward(xd, buf)).astype(np.float64)
    torch.cuda.synchronize()
    idx_gpu = _np(buf.topk_idx)
    # the permutation is exactly the permutation of the GPU's own indices
    off, perm_src, inv_pos = O.permute(idx_gpu, cfg.num_experts)
    np.testing.assert_array_equal(_np(buf.offsets), off)
    np.testing.assert_array_equal(_np(buf.perm_src), perm_src)
    np.testing.assert_array_equal(_np(buf.inv_pos), inv_pos)
    if n_sample is None:
        toks = np.arange(T)
    else:
        toks = np.unique(np.concatenate([[0, T - 1],
                                         np.random.default_rng(5).choice(T, n_sample, False)]))
    ref = checked_tokens(x[toks].astype(np.float64), wr, b, cfg.top_k, DeviceExperts(mats),
                         shared, idx_gpu[toks])
    err, bound = tol_check(out[toks], ref, f"{name} full-size output")
    print(f"[{name}] tokens checked {len(toks)}/{T}  max err {err:.3e} (bound {bound:.3e})")


@pytest.mark.parametrize("name,T,w8,gs", [
    ("decode_fine", 1, False, 128), ("decode_fine", 1, False, 64), ("decode_fine", 1, False, 256),
    ("decode_fine", 1, True, 128), ("decode_fine", 2, False, 128), ("decode_fine", 3, False, 128),
    ("decode_fine512", 1, False, 128), ("decode_fine512", 2, False, 128),
    ("decode_fine512", 4, False, 128), ("decode_coarse", 1, False, 128),
    ("decode_coarse", 1, False, 256)])
def test_full_size_small_batches(name, T, w8, gs):
    """Batches of a few tokens.  Where whole items would leave some CUs
    streaming two of them while others idle, the decode FFN splits each
    item's in_features over several blocks and adds their fp32 partial sums
    in a fixed order: the gate/up launch at one token on the 288-expert layer
    (quantization groups of 128, 64 and 256 columns), the down launch at one
    token on the coarse layer (groups of 128 and 256); the other cases run
    whole (the 8-bit shared expert is never split).  Every token against the
    oracle, after the permutation check."""
    cfg = get_config(name, tokens=T, group_size=gs)
    layer, mats, wr, b, shared = device_layer(cfg, w8=w8)
    x = G.activations(cfg, batch=20 + T)
    buf = layer.alloc(T)
    out = _np(layer.forward(torch.from_numpy(x).cuda(), buf)).astype(np.float64)
    torch.cuda.synchronize()
    idx_gpu = _np(buf.topk_idx)
    off, perm_src, inv_pos = O.permute(idx_gpu, cfg.num_experts)
    np.testing.assert_array_equal(_np(buf.offsets), off)
    np.testing.assert_array_equal(_np(buf.perm_src), perm_src)
    np.testing.assert_array_equal(_np(buf.inv_pos), inv_pos)
    ref = checked_tokens(x.astype(np.float64), wr, b, cfg.top_k, DeviceExperts(mats), shared,
                         idx_gpu)
    err, bound = tol_check(out, ref, f"{name} {T} token(s)")
    print(f"[{name} T={T}] max err {err:.3e} (bound {bound:.3e})")


def test_full_size_prefill_whole_segments():
    """The prefill layer at full shape (8192 tokens, 128 experts): every row
    of the FFN stage's output y_perm for whole segments: the largest, the
    smallest non-empty one, and the two whose last 128-row tile is the most
    and the least ragged, against the numpy oracle's expert FFN on the same
    rows; then segments of 1, 5 and 17 rows at the same shape (the layer's
    routing with a few choices moved to otherwise unchosen experts)."""
    cfg = get_config("prefill")
    layer, mats, wr, b, shared = device_layer(cfg)
    T, k = cfg.tokens, cfg.top_k
    x = G.activations(cfg, batch=0)
    buf = layer.alloc(T)
    layer.forward(torch.from_numpy(x).cuda(), buf)
    torch.cuda.synchronize()
    off = _np(buf.offsets).astype(np.int64)
    perm_src = _np(buf.perm_src).astype(np.int64)
    cnt = np.diff(off)
    live = np.nonzero(cnt > 0)[0]
    largest = int(live[np.argmax(cnt[live])])
    smallest = int(live[np.argmin(cnt[live])])
    long_ = [e for e in live if cnt[e] > 128 and cnt[e] % 128]
    most_ragged = int(max(long_, key=lambda e: (cnt[e] % 128, -e)))
    least_ragged = int(min(long_, key=lambda e: (cnt[e] % 128, e)))
    experts = DeviceExperts(mats)
    for what, e in (("largest", largest), ("smallest", smallest),
                    ("tail most ragged", most_ragged), ("tail least ragged", least_ragged)):
        r0, r1 = int(off[e]), int(off[e + 1])
        rows = x[perm_src[r0:r1] // k].astype(np.float64)
        ref = O.expert_ffn_w4(rows, *experts[e], group=cfg.group_size)
        got = _np(buf.y_perm[r0:r1]).astype(np.float64)
        err, bound = tol_check(got, ref, f"segment {e} ({what}, {r1 - r0} rows)")
        print(f"[prefill] {what} segment e={e}: {r1 - r0} rows (last tile {(r1 - r0) % 128 or 128}),"
              f" max err {err:.3e} (bound {bound:.3e})", flush=True)
        experts.cache.clear()
    # Near-empty segments at the same shape: the layer's routing with the last
    # choice of a few tokens moved to experts no token chose (segments of 1, 5
    # and 17 rows), then the permutation and the FFN stage on that routing.
    idx = _np(buf.topk_idx).copy()
    dead = [int(e) for e in np.nonzero(cnt == 0)[0]]
    assert len(dead) >= 3, "the prefill layer has experts no token chooses"
    t0 = 0
    for e, n in zip(dead, (1, 5, 17)):
        idx[t0:t0 + n, k - 1] = e
        t0 += n
    xd = torch.from_numpy(x).cuda()
    buf.topk_idx.copy_(torch.from_numpy(idx))
    layer.permute(xd, buf, T, gather=False)
    layer.ffn(xd, buf, T)
    torch.cuda.synchronize()
    off2, perm2, _ = O.permute(idx, cfg.num_experts)
    np.testing.assert_array_equal(_np(buf.offsets), off2)
    np.testing.assert_array_equal(_np(buf.perm_src), perm2)
    for e, n in zip(dead, (1, 5, 17)):
        r0, r1 = int(off2[e]), int(off2[e + 1])
        assert r1 - r0 == n
        rows = x[perm2[r0:r1].astype(np.int64) // k].astype(np.float64)
        ref = O.expert_ffn_w4(rows, *experts[e], group=cfg.group_size)
        err, bound = tol_check(_np(buf.y_perm[r0:r1]), ref, f"segment {e} ({n} rows)")
        print(f"[prefill] near-empty segment e={e}: {n} rows, max err {err:.3e} "
              f"(bound {bound:.3e})", flush=True)


@pytest.mark.parametrize("T", [16, 1])
def test_full_size_decode_stack(T):
    """42 layers, RMS norm between them, all 16 tokens (and one token: the
    K-split FFN in every layer), through
    moe_decode_stack_forward as the benchmark runs it (layer i's combine and
    layer i+1's routing in one launch).  A call over the first n layers must
    reproduce the full call's first n outputs bit for bit (its last combine is
    the standalone one) and leaves layer n-1's routing in the buffers, whose
    permutation must be exactly that of its selection.  Per layer,
    teacher-forced: the oracle's layer i runs on the GPU's fp16 input to layer
    i; its top-k must match under the tie rule and its RMS-normalised output
    (evaluated on the GPU's selection) must match the GPU's fp16 input to
    layer i+1 within the tolerance.  End to end: the oracle also carries its
    own float64 activations through all 42 layers; the final error is checked
    for the tokens whose routing never left the oracle's, and the routing
    flips are reported."""
    from w4_group_quantized_amd import W4MoEStack
    cfg = get_config("decode_stack", tokens=T)
    k = cfg.top_k
    layers = [device_layer(cfg, li) for li in range(cfg.layers)]
    stack = W4MoEStack([lay[0] for lay in layers])
    x = G.activations(cfg, batch=0)
    xd = torch.from_numpy(x).cuda()
    buf = stack.alloc(T)
    full = _np(stack.forward(xd, buf, rmsnorm=True, eps=cfg.rms_eps))
    idx_gpu = []
    for n in range(1, cfg.layers + 1):
        part = _np(stack.forward(xd, buf, rmsnorm=True, eps=cfg.rms_eps, n_layers=n))
        assert part.tobytes() == full[:n].tobytes(), f"first {n} layers differ from the full call"
        idx = _np(buf.topk_idx).copy()
        off, perm_src, inv_pos = O.permute(idx, cfg.num_experts)
        np.testing.assert_array_equal(_np(buf.offsets), off)
        np.testing.assert_array_equal(_np(buf.perm_src), perm_src)
        np.testing.assert_array_equal(_np(buf.inv_pos), inv_pos)
        idx_gpu.append(idx)
    acts = [x] + [full[li] for li in range(cfg.layers)]
    acts = [a.astype(np.float64) for a in acts]          # the GPU's fp16 layer inputs
    x_e2e = x.astype(np.float64)                         # the oracle's own activations
    alive = np.ones(T, dtype=bool)
    left_at = np.full(T, -1)
    worst = 0.0
    for li, (layer, mats, wr, b, shared) in enumerate(layers):
        experts = DeviceExperts(mats)
        # teacher-forced: the oracle's layer on the GPU's fp16 input
        y = checked_tokens(acts[li], wr, b, k, experts, shared, idx_gpu[li])
        err, bound = tol_check(acts[li + 1], O.rmsnorm(y, cfg.rms_eps), f"layer {li}")
        worst = max(worst, err / bound)
        # end to end on the oracle's own activations and routing
        y_e2e, idx_ref, _ = oracle_tokens(x_e2e, wr, b, k, experts, shared)
        same = (idx_ref == idx_gpu[li]).all(axis=1)
        left_at[alive & ~same] = li
        alive &= same
        x_e2e = O.rmsnorm(y_e2e, cfg.rms_eps)
        print(f"[decode_stack] layer {li}: teacher-forced max err {err:.3e} (bound {bound:.3e})",
              flush=True)
        del experts
    print(f"[decode_stack] per-layer worst err/bound {worst:.3f}; end to end: "
          f"{int((~alive).sum())} token(s) left the oracle's own routing (first layer where the "
          f"selections differ: {left_at.tolist()}), {int(alive.sum())}/{T} followed it through "
          f"all layers")
    if alive.any():
        err, bound = tol_check(acts[-1][alive], x_e2e[alive], "42-layer stack output")
        print(f"[decode_stack] end-to-end max err {err:.3e} (bound {bound:.3e})")
