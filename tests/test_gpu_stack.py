"""The stacked decode step, moe_decode_stack_forward: for up to 32 tokens the
combine of layer i and the router, top-k and permutation of layer i + 1 share
one launch (the output of one layer is the next layer's input:
haowenji.com/articles/x-2109226022155796480 §01).

Every layer is checked.  A call over the first n layers leaves layer n-1's
routing in the buffers and must reproduce the full call's first n outputs bit
for bit; its last combine runs as the standalone combine while the full call
fuses it with the next router, so this also shows that the fused launch's
rows are bitwise the combine's.  Layer n-1's selection is compared with the
oracle's under the tie rule, its permutation must be exactly the permutation
of that selection, and its output must match the oracle evaluated on the
GPU's selection and fp16 input to the layer (teacher-forced).
"""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from workloads import get_config
from workloads import gen as G

from gpu_util import (gpu, require_gpu, to_dev, tol_check, quantized_experts, coded_experts,
                      make_gpu_layer, on_gpu_selection, shared_w8)

pytestmark = gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _np(t):
    return t.detach().cpu().numpy()


def oracle_layer(x, wr, b, experts, cfg, shared, idx=None):
    return O.moe_layer(x, wr, b, experts, cfg.top_k, shared=shared,
                       expert_ffn=functools.partial(O.expert_ffn_w4, group=cfg.group_size),
                       idx=idx)


def build_stack(cfg, n_layers, w8=False):
    from w4_group_quantized_amd import W4MoEStack
    layers, refs = [], []
    for li in range(n_layers):
        mats, experts = quantized_experts(cfg, layer=li)
        wr, b = G.router(cfg, li)
        shared = G.shared_expert(cfg, li)
        if w8 and shared is not None:
            stored, deq = shared_w8(shared)
            layers.append(make_gpu_layer(cfg, mats, wr, b, None, w8=stored))
            refs.append((wr, b, experts, deq))
        else:
            layers.append(make_gpu_layer(cfg, mats, wr, b, shared))
            refs.append((wr, b, experts, shared))
    return W4MoEStack(layers), layers, refs


def check_stack(cfg, n_layers, T, rmsnorm=True, renorm=False, w8=False, batch=0):
    stack, layers, refs = build_stack(cfg, n_layers, w8=w8)
    k = cfg.top_k
    x = G.activations(cfg, tokens=T, batch=batch)
    xd = to_dev(x)
    buf = stack.alloc(T)
    kw = dict(rmsnorm=rmsnorm, eps=cfg.rms_eps, renorm=renorm)
    acts = _np(stack.forward(xd, buf, **kw))
    torch.cuda.synchronize()
    for n in range(1, n_layers + 1):
        part = _np(stack.forward(xd, buf, n_layers=n, **kw))
        assert part.tobytes() == acts[:n].tobytes(), f"first {n} layers differ from the full call"
        li = n - 1
        xin = x if li == 0 else acts[li - 1]
        wr, b, experts, sh = refs[li]
        idx = _np(buf.topk_idx)[:T]
        off, perm_src, inv_pos = O.permute(idx, cfg.num_experts)
        np.testing.assert_array_equal(_np(buf.offsets), off)
        np.testing.assert_array_equal(_np(buf.perm_src)[:T * k], perm_src)
        np.testing.assert_array_equal(_np(buf.inv_pos)[:T * k], inv_pos)
        ref = on_gpu_selection(oracle_layer(xin, wr, b, experts, cfg, sh), idx,
                               lambda i: oracle_layer(xin, wr, b, experts, cfg, sh, idx=i), k)
        np.testing.assert_allclose(_np(buf.topk_w)[:T], ref["w"], rtol=1e-5, atol=1e-7)
        y = O.combine(ref["y_perm"], ref["ys"], ref["inv_pos"], ref["w"], T, k, renorm=renorm)
        if rmsnorm:
            y = O.rmsnorm(y, cfg.rms_eps)
        tol_check(acts[li], y, f"{cfg.name} stack layer {li}")
    return stack, layers, acts


FINE = dict(num_experts=48, hidden=512, ffn=256, shared_ffn=256)


@pytest.mark.parametrize("T", [1, 5, 16, 32])
def test_stack_fine_grained_scaled_down(T):
    """48 experts + shared, hidden 512, ffn 256, top-8, 4 layers, RMS norm."""
    check_stack(get_config("decode_fine", **FINE), 4, T, batch=T)


def test_stack_without_norm_and_with_renormalised_weights():
    cfg = get_config("decode_fine", **FINE)
    check_stack(cfg, 3, 13, rmsnorm=False, batch=2)
    check_stack(cfg, 3, 9, rmsnorm=True, renorm=True, batch=3)


def test_stack_group_size_64_and_8bit_shared_expert():
    check_stack(get_config("decode_fine", group_size=64, **FINE), 3, 7, batch=4)
    check_stack(get_config("decode_fine", **FINE), 3, 16, w8=True, batch=5)


WIDE = dict(num_experts=4, hidden=8192, ffn=256, top_k=2, shared_ffn=256)


@pytest.mark.parametrize("T,dims", [(10, "fine"), (1, "wide"), (3, "wide")])
def test_stack_mixed_group_sizes_and_shared_formats(T, dims):
    """Layers of one stack may differ in group size and in the shared
    expert's format (only the shapes must agree).  On the hidden-8192 layers
    at 1 and 3 tokens the layers with the fp16 shared expert split their
    gate/up items in K over blocks and the one with the 8-bit shared expert
    does not, all in one workspace, between fused combine + router launches
    (expert weights drawn as codes)."""
    from w4_group_quantized_amd import W4MoEStack
    wide = dims == "wide"
    cfgs = [get_config("decode_fine", group_size=gs, **(WIDE if wide else FINE))
            for gs in (128, 64, 256)]
    layers, refs = [], []
    for li, cfg in enumerate(cfgs):
        mats, experts = (coded_experts if wide else quantized_experts)(cfg, layer=li)
        wr, b = G.router(cfg, li)
        shared = G.shared_expert(cfg, li)
        if li == 1:
            stored, deq = shared_w8(shared)
            layers.append(make_gpu_layer(cfg, mats, wr, b, None, w8=stored))
            refs.append((cfg, wr, b, experts, deq))
        else:
            layers.append(make_gpu_layer(cfg, mats, wr, b, shared))
            refs.append((cfg, wr, b, experts, shared))
    stack = W4MoEStack(layers)
    x = G.activations(cfgs[0], tokens=T, batch=11)
    buf = stack.alloc(T)
    acts = _np(stack.forward(to_dev(x), buf, eps=cfgs[0].rms_eps))
    for n in range(1, len(layers) + 1):
        part = _np(stack.forward(to_dev(x), buf, eps=cfgs[0].rms_eps, n_layers=n))
        assert part.tobytes() == acts[:n].tobytes()
        cfg, wr, b, experts, sh = refs[n - 1]
        xin = x if n == 1 else acts[n - 2]
        idx = _np(buf.topk_idx)[:T]
        ref = on_gpu_selection(oracle_layer(xin, wr, b, experts, cfg, sh), idx,
                               lambda i: oracle_layer(xin, wr, b, experts, cfg, sh, idx=i),
                               cfg.top_k)
        tol_check(acts[n - 1], O.rmsnorm(ref["out"], cfg.rms_eps), f"mixed stack layer {n - 1}")


def test_stack_without_shared_expert():
    """16 experts, top-4, no shared expert (the coarse layer's routing law)."""
    check_stack(get_config("decode_coarse", num_experts=16, hidden=512, ffn=256, top_k=4), 3, 16,
                batch=6)


@pytest.mark.parametrize("E,k,T", [(288, 8, 16), (288, 8, 32), (1024, 32, 4), (40, 1, 11),
                                   (1024, 32, 1), (40, 1, 1), (288, 8, 1), (16, 16, 1)])
def test_stack_expert_tiles(E, k, T):
    """Expert tiles sized to give every CU one block: 288 experts at 16
    tokens (18 per block, 16 tiles, two per XCD) and at 32 (36 per block, 8
    tiles, more than one expert per wave), 1024 experts at top-32 (16 per
    block, 64 tiles), and top-1 over 40 experts; at one token (the token's
    own block sorts its choices into the permutation) top-32 of 1024, top-1
    of 40, top-8 of 288 and every expert (top-16 of 16)."""
    cfg = get_config("decode_fine", num_experts=E, hidden=256, ffn=128, top_k=k, shared_ffn=128)
    check_stack(cfg, 3, T, batch=7 + T)


def test_stack_of_one_layer_is_the_layer_call():
    cfg = get_config("decode_fine", **FINE)
    stack, layers, acts = check_stack(cfg, 1, 12, batch=8)
    x = to_dev(G.activations(cfg, tokens=12, batch=8))
    buf = layers[0].alloc(12)
    out = _np(layers[0].forward(x, buf, rmsnorm=True, eps=cfg.rms_eps))
    assert out.tobytes() == acts[0].tobytes()


def test_stack_above_32_tokens_is_the_layer_calls():
    """Past 32 tokens each layer runs as moe_layer_forward does, bitwise."""
    cfg = get_config("decode_fine", **FINE)
    T = 40
    stack, layers, acts = check_stack(cfg, 3, T, batch=9)
    x = to_dev(G.activations(cfg, tokens=T, batch=9))
    buf = layers[0].alloc(T)
    a = x
    for li, layer in enumerate(layers):
        out = torch.empty_like(x)
        layer.forward(a, buf, rmsnorm=True, eps=cfg.rms_eps, out=out)
        torch.cuda.synchronize()
        assert _np(out).tobytes() == acts[li].tobytes(), f"layer {li}"
        a = out


def test_stack_repeated_calls_bitwise():
    """The fused launches leave their counters at zero: 200 calls in a row
    give the first call's outputs and routing, bit for bit."""
    cfg = get_config("decode_fine", num_experts=288, hidden=512, ffn=256, shared_ffn=256)
    stack, _, _ = build_stack(cfg, 3)
    T = 16
    x = to_dev(G.activations(cfg, tokens=T, batch=10))
    buf = stack.alloc(T)
    first = stack.forward(x, buf).clone()
    idx0 = buf.topk_idx.clone()
    n = 200
    hist = torch.empty((n,) + tuple(first.shape), dtype=first.dtype, device=x.device)
    ihist = torch.empty((n,) + tuple(idx0.shape), dtype=idx0.dtype, device=x.device)
    acts = torch.empty_like(first)
    for i in range(n):
        stack.forward(x, buf, acts=acts)
        hist[i].copy_(acts)
        ihist[i].copy_(buf.topk_idx)
    torch.cuda.synchronize()
    same = (hist.view(n, -1).view(torch.int16) == first.view(1, -1).view(torch.int16)).all(dim=1)
    same &= (ihist.view(n, -1) == idx0.view(1, -1)).all(dim=1)
    bad = torch.nonzero(~same)
    assert bad.numel() == 0, f"call {int(bad[0])} of {n} differs from the first"
