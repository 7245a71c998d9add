"""moe_layer_forward_noalloc (the whole-layer call whose workspace is a fixed
array inside the library) against moe_layer_forward (caller's workspace):
every output bitwise equal, on consecutive calls of which the later one is
smaller, at a scaled-down decode shape and at the full 288-expert decode
shape; and the host-side refusal of a layer whose workspace would not fit.
"""
import ctypes

import pytest
import torch

import oracle as O
from workloads import get_config
from workloads import gen as G
from workloads import gen_torch as GT

from gpu_util import gpu, require_gpu, to_dev, tol_check, quantized_experts, make_gpu_layer

N = pytest.importorskip("w4_group_quantized_amd._native",
                        reason="libmoe_w4.so not built (python w4_group_quantized_amd/build.py)")

OUTS = ("topk_idx", "topk_w", "offsets", "perm_src", "inv_pos", "y_perm", "y_shared", "out")


def _np(t):
    return t.detach().cpu().numpy()


def noalloc_forward(layer, x, buf, T, rmsnorm=False, eps=1e-6):
    flags = N.MOE_RMSNORM if rmsnorm else 0
    N.moe_layer_forward_noalloc(layer.desc, x, T, buf.topk_idx, buf.topk_w, buf.offsets,
                                buf.perm_src, buf.inv_pos, None, buf.y_perm,
                                buf.y_shared if layer.Fs else None, flags, eps, buf.out)


def compare(layer, buf_ref, buf_na, T):
    k = layer.k
    rows = {"topk_idx": T, "topk_w": T, "offsets": None, "perm_src": T * k, "inv_pos": T * k,
            "y_perm": T * k, "y_shared": T, "out": T}
    for n in OUTS:
        a, b = getattr(buf_ref, n), getattr(buf_na, n)
        if rows[n] is not None:
            a, b = a[:rows[n]], b[:rows[n]]
        assert _np(a).tobytes() == _np(b).tobytes(), f"T={T}: {n} differs"


@gpu
def test_noalloc_matches_layer_forward_scaled_down():
    require_gpu()
    cfg = get_config("decode_fine", num_experts=48, hidden=512, ffn=256, shared_ffn=256)
    mats, experts = quantized_experts(cfg)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    layer = make_gpu_layer(cfg, mats, wr, b, shared)
    buf_ref, buf_na = layer.alloc(13), layer.alloc(13)
    for T in (13, 5):                                 # the second call is smaller
        x = G.activations(cfg, tokens=T, batch=80 + T)
        xd = to_dev(x)
        layer.forward(xd, buf_ref, T)
        noalloc_forward(layer, xd, buf_na, T)
        torch.cuda.synchronize()
        compare(layer, buf_ref, buf_na, T)
        ref = O.moe_layer(x, wr, b, experts, cfg.top_k, shared=shared,
                          idx=_np(buf_na.topk_idx)[:T])
        differs, excused = O.tie_excused(_np(buf_na.topk_idx)[:T], ref["logits"])
        assert not (differs & ~excused).any()
        tol_check(_np(buf_na.out)[:T], ref["out"], f"T={T} out")


@gpu
def test_noalloc_matches_layer_forward_full_decode_shape():
    """288 experts + shared expert, hidden 4096, ffn 1536, top-8: 16, 8, then
    1 token (whose FFN keeps its K-split partial sums and tickets in the fixed
    array), with the RMS norm of the stacked layers."""
    require_gpu()
    from w4_group_quantized_amd import W4MoELayer
    cfg = get_config("decode_stack", layers=1)
    dev = torch.device("cuda:0")
    mats = GT.layer_codes(cfg, 0, dev)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    layer = W4MoELayer(cfg.top_k, to_dev(wr), to_dev(b), mats["gate_q"], mats["gate_s"],
                       mats["up_q"], mats["up_s"], mats["down_q"], mats["down_s"],
                       shared=tuple(to_dev(w) for w in shared))
    buf_ref, buf_na = layer.alloc(16), layer.alloc(16)
    for T in (16, 8, 1):
        xd = to_dev(G.activations(cfg, tokens=T, batch=90 + T))
        layer.forward(xd, buf_ref, T, rmsnorm=True, eps=cfg.rms_eps)
        noalloc_forward(layer, xd, buf_na, T, rmsnorm=True, eps=cfg.rms_eps)
        torch.cuda.synchronize()
        compare(layer, buf_ref, buf_na, T)


def test_noalloc_refuses_what_does_not_fit():
    """Checked on the host before any launch: the 8192-token prefill layer
    needs a 262 MiB workspace; null pointers are refused first."""
    FAKE = 1 << 20
    cfg = get_config("prefill")
    L = N.make_layer(num_experts=cfg.num_experts, hidden=cfg.hidden, ffn=cfg.ffn,
                     top_k=cfg.top_k, router_w=FAKE, router_b=None, gate_q=FAKE, gate_s=FAKE,
                     up_q=FAKE, up_s=FAKE, down_q=FAKE, down_s=FAKE)
    f = N.lib.moe_layer_forward_noalloc
    # topk_idx, topk_w, offsets, perm_src, inv_pos, x_perm, y_perm, y_shared, flags, eps, out,
    # stream
    args = [FAKE] * 5 + [None, FAKE, None, 0, ctypes.c_float(1e-6), FAKE, None]
    assert f(ctypes.byref(L), FAKE, 8192, *args) == -3              # MOE_EWORKSPACE
    assert f(ctypes.byref(L), None, 8192, *args) == -1              # MOE_EINVAL
    assert f(ctypes.byref(L), FAKE, 0, *args) == 0                  # T = 0: nothing to do
