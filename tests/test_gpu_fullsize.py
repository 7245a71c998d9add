"""Full-size parity in the launch configuration the benchmark times
(moe_route_permute -> moe_w4_grouped_ffn reading rows through perm_src ->
moe_unpermute_combine), against the float64 oracle on sampled tokens (every
token of the decode workloads).  Tokens are independent in an MoE layer, so
sampled outputs are checked exactly as in a full run.  Expert weights are
packed codes + scales drawn directly on the device; the oracle reads back the
experts it needs and evaluates them with the C reference products."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import cref as C
from workloads import get_config
from workloads import gen as G
from workloads import gen_torch as GT

from gpu_util import gpu, require_gpu, tol_check, route_compare

pytestmark = gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _np(t):
    return t.detach().cpu().numpy()


def device_layer(cfg, layer_idx=0):
    from w4_group_quantized_amd import W4MoELayer
    dev = torch.device("cuda:0")
    mats = GT.layer_codes(cfg, layer_idx, dev)
    wr, b = G.router(cfg, layer_idx)
    shared = G.shared_expert(cfg, layer_idx)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    layer = W4MoELayer(cfg.top_k, t(wr), t(b) if b is not None else None, mats["gate_q"],
                       mats["gate_s"], mats["up_q"], mats["up_s"], mats["down_q"], mats["down_s"],
                       shared=tuple(t(w) for w in shared) if shared is not None else None)
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


def oracle_tokens(x64, wr, b, k, experts, shared):
    """Float64 layer output for the given token rows (token-independent)."""
    idx, w, logits = O.route(x64, wr, b, k)
    out = O.swiglu_ffn(x64, *shared) if shared is not None else np.zeros((x64.shape[0], wr.shape[1]))
    for e in np.unique(idx):
        rows, slots = np.nonzero(idx == e)
        y = C.expert_ffn_w4_c(x64[rows], *experts[e])
        out[rows] += w[rows, slots][:, None] * y
    return out, idx, logits


@pytest.mark.parametrize("name,n_sample", [("decode_fine", None), ("decode_coarse", None),
                                           ("prefill", 48), ("decode_fine512", None)])
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
    ref, idx_ref, logits = oracle_tokens(x[toks].astype(np.float64), wr, b, cfg.top_k,
                                         DeviceExperts(mats), shared)
    diff = route_compare(idx_gpu[toks], idx_ref, logits, cfg.top_k)
    ok = ~diff
    err, bound = tol_check(out[toks][ok], ref[ok], f"{name} full-size output")
    print(f"[{name}] tokens checked {int(ok.sum())}/{len(toks)}  max err {err:.3e} (bound {bound:.3e})")


def test_full_size_decode_stack():
    """42 layers, RMS norm between them, on the device end to end; the oracle
    follows two tokens through all layers in float64 (no fp16 rounding of the
    activations).  A token whose routing meets a reported near tie on the way
    is not compared after it (routing is discrete)."""
    cfg = get_config("decode_stack")
    T = cfg.tokens
    layers = [device_layer(cfg, l) for l in range(cfg.layers)]
    x = G.activations(cfg, batch=0)
    xd = torch.from_numpy(x).cuda()
    buf = layers[0][0].alloc(T)
    act = [torch.empty_like(xd), torch.empty_like(xd)]
    cur = xd
    idx_gpu = []
    for li, (layer, *_r) in enumerate(layers):
        nxt = act[li % 2]
        layer.forward(cur, buf, rmsnorm=True, eps=cfg.rms_eps, out=nxt)
        idx_gpu.append(_np(buf.topk_idx).copy())
        cur = nxt
    out = _np(cur).astype(np.float64)
    toks = np.array([0, T - 1])
    x64 = x[toks].astype(np.float64)
    alive = np.ones(len(toks), dtype=bool)
    for li, (layer, mats, wr, b, shared) in enumerate(layers):
        y, idx_ref, logits = oracle_tokens(x64, wr, b, cfg.top_k, DeviceExperts(mats), shared)
        same = (idx_gpu[li][toks] == idx_ref).all(axis=1)
        ties = O.near_ties(logits, cfg.top_k)
        assert (same | ties | ~alive).all(), f"layer {li}: top-k differs away from a near tie"
        alive &= same
        x64 = O.rmsnorm(y, cfg.rms_eps)
    assert alive.any(), "every sampled token met a near tie"
    err, bound = tol_check(out[toks][alive], x64[alive], "42-layer stack output")
    print(f"[decode_stack] tokens {int(alive.sum())}/{len(toks)} max err {err:.3e} (bound {bound:.3e})")
