"""Repeated and captured execution.

The one-launch router and permutation hands its partial logits across the
XCDs through a device-wide completion counter that every call leaves at zero:
a thousand back-to-back calls must all give the first call's outputs, bit for
bit, and that first call must match the oracle.  A layer and the 42-layer
decode step captured into HIP graphs must replay bitwise equal to eager
execution (the pages capture the grouped expert GEMM into a fixed graph:
xdnf.cn/news/329730 §3.2, §4.3), with the program's own eager work between
replays.
"""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import get_config
from workloads import gen as G
from workloads import gen_torch as GT

from gpu_util import gpu, require_gpu, to_dev, route_compare

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
    return W4MoELayer(cfg.top_k, t(wr), t(b) if b is not None else None, mats["gate_q"],
                      mats["gate_s"], mats["up_q"], mats["up_s"], mats["down_q"], mats["down_s"],
                      shared=tuple(t(w) for w in shared) if shared is not None else None)


ROUTING = ("topk_idx", "topk_w", "offsets", "perm_src", "inv_pos")


@pytest.mark.parametrize("T", [8, 16, 28, 64])
def test_route_permute_thousand_calls_bitwise_stable(T):
    """The 288-expert router (one launch up to 28 tokens, where T * E fits
    the last block's LDS; separate router and permutation launches at 64)."""
    from w4_group_quantized_amd import W4MoELayer
    cfg = get_config("decode_fine")
    wr, b = G.router(cfg)
    z8 = to_dev(np.zeros((1, 1, 16), np.uint8))
    z16 = to_dev(np.zeros((1, 1, 8), np.float16))
    layer = W4MoELayer(cfg.top_k, to_dev(wr), to_dev(b), z8, z16, z8, z16, z8, z16,
                       group_size=cfg.group_size)
    layer.desc.ffn = cfg.ffn
    x = G.activations(cfg, tokens=T, batch=50 + T)
    xd = to_dev(x)
    buf = layer.alloc(T)
    layer.route_permute(xd, buf, T)
    torch.cuda.synchronize()
    idx = _np(buf.topk_idx)
    _, _, logits = O.route(x, wr, b, cfg.top_k)
    route_compare(idx, logits, cfg.top_k)
    off, perm_src, inv_pos = O.permute(idx, cfg.num_experts)
    assert (_np(buf.offsets) == off).all() and (_np(buf.perm_src) == perm_src).all()
    assert (_np(buf.inv_pos) == inv_pos).all()
    first = {n: getattr(buf, n).clone() for n in ROUTING}
    n_calls = 1000
    hist = {n: torch.empty((n_calls,) + tuple(first[n].shape), dtype=first[n].dtype,
                           device=xd.device) for n in ROUTING}
    for i in range(n_calls):
        layer.route_permute(xd, buf, T)
        for n in ROUTING:
            hist[n][i].copy_(getattr(buf, n))
    torch.cuda.synchronize()
    for n in ROUTING:
        same = (hist[n].view(n_calls, -1) == first[n].view(1, -1)).all(dim=1) if n != "topk_w" \
            else (hist[n].view(n_calls, -1).view(torch.int32) ==
                  first[n].view(1, -1).view(torch.int32)).all(dim=1)
        bad = torch.nonzero(~same)
        assert bad.numel() == 0, f"{n}: call {int(bad[0])} of {n_calls} differs from the first"


@pytest.mark.parametrize("name,T", [("decode_fine", 1), ("decode_coarse", 1)])
def test_split_ffn_repeated_calls_bitwise(name, T):
    """The decode FFN's K-split blocks hand their partial sums across the XCDs
    through per-item tickets that every call leaves at zero: 300 whole-layer
    calls in a row give the first call's outputs bit for bit."""
    cfg = get_config(name, tokens=T)
    layer = device_layer(cfg)
    x = to_dev(G.activations(cfg, batch=70 + T))
    buf = layer.alloc(T)
    first = layer.forward(x, buf).clone()
    n_calls = 300
    hist = torch.empty((n_calls,) + tuple(first.shape), dtype=first.dtype, device=x.device)
    for i in range(n_calls):
        hist[i].copy_(layer.forward(x, buf))
    torch.cuda.synchronize()
    same = (hist.view(n_calls, -1).view(torch.int16) ==
            first.view(1, -1).view(torch.int16)).all(dim=1)
    bad = torch.nonzero(~same)
    assert bad.numel() == 0, f"call {int(bad[0])} of {n_calls} differs from the first"


def _replay_check(g, static_out, eager_out, eager_work, replays=4):
    for r in range(replays):
        eager_work()                     # the program's own eager launches in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got in static_out.items():
            assert _np(got).tobytes() == eager_out[name], f"replay {r}: {name} differs"


@pytest.mark.parametrize("T", [1, 8, 16])
def test_layer_graph_replay_bitwise(T):
    """moe_layer_forward at the fine-grained decode shape (288 experts + shared,
    hidden 4096, ffn 1536) captured once, replayed four times (at one token
    with the FFN's K split over blocks and its per-item tickets)."""
    cfg = get_config("decode_fine", tokens=T)
    layer = device_layer(cfg)
    x = to_dev(G.activations(cfg, batch=60 + T))
    x_other = to_dev(G.activations(cfg, batch=61 + T))
    buf = layer.alloc(T)
    other = layer.alloc(T)
    layer.forward(x, buf)
    torch.cuda.synchronize()
    names = ROUTING + ("y_perm", "y_shared", "out")
    eager = {n: _np(getattr(buf, n)).tobytes() for n in names}
    for n in names:
        getattr(buf, n).zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, buf)
    _replay_check(g, {n: getattr(buf, n) for n in names}, eager,
                  lambda: layer.forward(x_other, other))


def test_decode_stack_graph_replay_bitwise():
    """The 42-layer decode step (RMS norm between layers) captured into one
    graph: every layer's output after each replay equals eager execution."""
    cfg = get_config("decode_stack")
    T = cfg.tokens
    layers = [device_layer(cfg, li) for li in range(cfg.layers)]
    x = to_dev(G.activations(cfg, batch=70))
    buf = layers[0].alloc(T)
    acts = [x] + [torch.empty_like(x) for _ in range(cfg.layers)]

    def step(a, bf):
        for li, layer in enumerate(layers):
            layer.forward(a[li], bf, rmsnorm=True, eps=cfg.rms_eps, out=a[li + 1])

    step(acts, buf)
    torch.cuda.synchronize()
    eager = {f"layer {li}": _np(acts[li + 1]).tobytes() for li in range(cfg.layers)}
    for a in acts[1:]:
        a.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(acts, buf)
    other_acts = [to_dev(G.activations(cfg, batch=71))] + [torch.empty_like(x)
                                                           for _ in range(cfg.layers)]
    other_buf = layers[0].alloc(T)
    _replay_check(g, {f"layer {li}": acts[li + 1] for li in range(cfg.layers)}, eager,
                  lambda: step(other_acts, other_buf), replays=3)


@pytest.mark.parametrize("T", [16, 1])
def test_decode_stack_call_graph_replay_bitwise(T):
    """moe_decode_stack_forward over the 42 layers (the fused combine + next
    router launches) captured into one graph: every layer's output and the
    last layer's routing after each replay equal eager execution (at one
    token: the K-split gate/up launch and the one-token permutation)."""
    from w4_group_quantized_amd import W4MoEStack
    cfg = get_config("decode_stack", tokens=T)
    stack = W4MoEStack([device_layer(cfg, li) for li in range(cfg.layers)])
    x = to_dev(G.activations(cfg, batch=72))
    buf = stack.alloc(T)
    acts = torch.empty((cfg.layers, T, cfg.hidden), dtype=torch.float16, device=x.device)
    stack.forward(x, buf, acts=acts, eps=cfg.rms_eps)
    torch.cuda.synchronize()
    names = ("topk_idx", "topk_w", "offsets", "perm_src", "inv_pos")
    eager = {"acts": _np(acts).tobytes()}
    eager.update({n: _np(getattr(buf, n)).tobytes() for n in names})
    acts.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack.forward(x, buf, acts=acts, eps=cfg.rms_eps)
    other_x = to_dev(G.activations(cfg, batch=73))
    other_buf = stack.alloc(T)
    static = {"acts": acts}
    static.update({n: getattr(buf, n) for n in names})
    _replay_check(g, static, eager, lambda: stack.forward(other_x, other_buf, eps=cfg.rms_eps),
                  replays=3)
