"""End-to-end parity of one MoE layer forward (route -> permute -> grouped FFN
-> combine, all through the C ABI) against the float64 oracle."""
import functools

import numpy as np
import pytest
import torch

import oracle as O
from workloads import get_config
from workloads import gen as G

from gpu_util import (gpu, require_gpu, to_dev, tol_check, quantized_experts, coded_experts,
                      make_gpu_layer, on_gpu_selection)

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


def check_selection(ref, buf, T, x, wr, b, experts, cfg, shared):
    """Indices under the tie rule; the oracle on the GPU's selection when they
    differ; the permutation always bit-exact."""
    ref = on_gpu_selection(ref, _np(buf.topk_idx)[:T],
                           lambda idx: oracle_layer(x, wr, b, experts, cfg, shared, idx=idx),
                           cfg.top_k)
    np.testing.assert_array_equal(_np(buf.offsets), ref["offsets"])
    np.testing.assert_array_equal(_np(buf.perm_src)[:T * cfg.top_k], ref["perm_src"])
    np.testing.assert_array_equal(_np(buf.inv_pos)[:T * cfg.top_k], ref["inv_pos"])
    return ref


def run_layer_case(cfg, T, batch=0, separate_calls=False):
    mats, experts = quantized_experts(cfg)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    x = G.activations(cfg, tokens=T, batch=batch)
    ref = oracle_layer(x, wr, b, experts, cfg, shared)
    layer = make_gpu_layer(cfg, mats, wr, b, shared)
    buf = layer.alloc(T)
    xd = to_dev(x)
    if separate_calls:       # the four calls of the boundary, x_perm materialised
        layer.route(xd, buf, T)
        layer.permute(xd, buf, T, gather=True)
        layer.ffn(xd, buf, T, use_x_perm=True)
        layer.combine(buf, T)
        out = buf.out
    else:
        out = layer.forward(xd, buf)
    torch.cuda.synchronize()
    ref = check_selection(ref, buf, T, x, wr, b, experts, cfg, shared)
    tol_check(_np(out), ref["out"], f"{cfg.name} out")
    return layer, buf, x


@pytest.mark.parametrize("separate_calls", [False, True])
def test_tiny_layer_exact_config(separate_calls):
    """8 experts, hidden 256, ffn 512, top-2, 16 tokens, seed 0."""
    run_layer_case(get_config("tiny"), 16, separate_calls=separate_calls)


@pytest.mark.parametrize("T", [1, 8, 13])
def test_fine_grained_shape_scaled_down(T):
    cfg = get_config("decode_fine", num_experts=48, hidden=512, ffn=256, shared_ffn=256)
    run_layer_case(cfg, T, batch=T)


@pytest.mark.parametrize("separate_calls", [False, True])
def test_prefill_like_ragged_segments(separate_calls):
    cfg = get_config("prefill", num_experts=16, hidden=256, ffn=384, top_k=4)
    run_layer_case(cfg, 150, separate_calls=separate_calls)


def test_largest_expert_count_and_top_k():
    """1024 experts, top-32, 4 tokens: the tile lookups over 1024 segments and
    32 rows of y_perm per token in the combine."""
    cfg = get_config("decode_fine", num_experts=1024, hidden=256, ffn=128, top_k=32,
                     shared_ffn=128)
    run_layer_case(cfg, 4, batch=9)


def test_layer_is_deterministic():
    cfg = get_config("decode_fine", num_experts=32, hidden=384, ffn=256, shared_ffn=128)
    layer, buf, x = run_layer_case(cfg, 11)
    first = _np(buf.out).copy()
    for _ in range(3):
        layer.forward(to_dev(x), buf)
    torch.cuda.synchronize()
    assert _np(buf.out).tobytes() == first.tobytes()


def test_zero_tokens_is_a_noop():
    cfg = get_config("tiny")
    mats, _ = quantized_experts(cfg, experts=range(cfg.num_experts))
    wr, b = G.router(cfg)
    layer = make_gpu_layer(cfg, mats, wr, b, None)
    buf = layer.alloc(4)
    buf.out.fill_(7)
    x = to_dev(G.activations(cfg, tokens=4))
    layer.forward(x[:0], buf, T=0)
    torch.cuda.synchronize()
    assert (_np(buf.out) == 7).all()


@pytest.mark.parametrize("E,H,F,k,T", [(16, 256, 384, 4, 150), (8, 512, 256, 2, 700),
                                       (32, 768, 384, 8, 300)])
def test_prefill_kernel_path(E, H, F, k, T):
    """Average segment >= 32 rows and H % 256 == 0: the LDS-tiled MFMA path,
    with ragged segment tails (segments not multiples of 128 rows)."""
    cfg = get_config("prefill", num_experts=E, hidden=H, ffn=F, top_k=k, dead_experts=1)
    run_layer_case(cfg, T, batch=3)


@pytest.mark.parametrize("gs,E,H,F,k,T", [(64, 16, 256, 384, 4, 150), (256, 8, 512, 256, 2, 700),
                                          (64, 32, 768, 384, 8, 300)])
def test_prefill_kernel_path_group_sizes(gs, E, H, F, k, T):
    """The MFMA prefill path with 64- and 256-column groups (its scale of a
    64-column K step is group step, step / 2 or step / 4)."""
    cfg = get_config("prefill", num_experts=E, hidden=H, ffn=F, top_k=k, dead_experts=1,
                     group_size=gs)
    run_layer_case(cfg, T, batch=4)


@pytest.mark.parametrize("gs", [64, 256])
def test_decode_layer_group_sizes(gs):
    """A fine-grained decode layer (one-launch router, shared expert) with
    64- and 256-column groups."""
    cfg = get_config("decode_fine", num_experts=48, hidden=512, ffn=256, shared_ffn=256,
                     group_size=gs)
    run_layer_case(cfg, 8, batch=gs)


def test_one_workspace_for_calls_of_different_sizes():
    """Buffers and workspace allocated once for the largest call, then calls of
    growing and shrinking T in turn: the fused router (T <= 64), the
    separate router and permutation, and the MFMA prefill path (T >= 128 here)
    must each find what they need, with no state left over from the calls
    before."""
    cfg = get_config("prefill", num_experts=16, hidden=256, ffn=384, top_k=4, shared_ffn=128)
    mats, experts = quantized_experts(cfg)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    layer = make_gpu_layer(cfg, mats, wr, b, shared)
    buf = layer.alloc(700)
    for T in (13, 1, 700, 8, 64, 65, 0, 150, 5):
        x = G.activations(cfg, tokens=max(T, 1), batch=T)[:T]
        out = layer.forward(to_dev(x), buf, T=T)
        torch.cuda.synchronize()
        if T == 0:
            continue
        ref = oracle_layer(x, wr, b, experts, cfg, shared)
        ref = check_selection(ref, buf, T, x, wr, b, experts, cfg, shared)
        tol_check(_np(out), ref["out"], f"T={T} out")


@pytest.mark.parametrize("E,H,F,Fs,k,T,gather", [
    (48, 512, 256, 256, 8, 8, False),     # one-launch router
    (48, 384, 256, 384, 4, 40, False),    # three token tiles
    (32, 256, 128, 0, 2, 5, False),       # no shared expert
    (16, 256, 384, 128, 4, 64, True),     # the largest one-launch batch, x_perm written
    (16, 256, 384, 128, 4, 150, False),   # separate router and permutation launches
    (16, 256, 384, 128, 4, 150, True),
    (128, 1024, 256, 512, 8, 64, False),  # T*E = 8192 logits: the one-launch limit
])
def test_forward_matches_staged_calls(E, H, F, Fs, k, T, gather):
    """moe_layer_forward against moe_route_permute + moe_w4_grouped_ffn +
    moe_unpermute_combine on the same inputs: every output bitwise equal, and
    the layer output within the oracle tolerance."""
    cfg = get_config("decode_fine", num_experts=E, hidden=H, ffn=F, top_k=k, shared_ffn=Fs)
    mats, experts = quantized_experts(cfg)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    x = G.activations(cfg, tokens=T, batch=T)
    ref = O.moe_layer(x, wr, b, experts, cfg.top_k, shared=shared)
    layer = make_gpu_layer(cfg, mats, wr, b, shared)
    b1, b2 = layer.alloc(T), layer.alloc(T)
    xd = to_dev(x)
    layer.forward(xd, b1, gather=gather)
    layer.forward_staged(xd, b2, gather=gather)
    torch.cuda.synchronize()
    names = ["topk_idx", "topk_w", "offsets", "perm_src", "inv_pos", "y_perm", "y_shared", "out"]
    if gather:
        names.append("x_perm")
    for name in names:
        assert _np(getattr(b1, name)).tobytes() == _np(getattr(b2, name)).tobytes(), name
    ref = check_selection(ref, b1, T, x, wr, b, experts, cfg, shared)
    if gather:
        assert _np(b1.x_perm).tobytes() == np.asarray(ref["x_perm"], np.float16).tobytes()
    tol_check(_np(b1.out), ref["out"], "out")


def test_forward_into_separate_output_with_norm():
    """moe_layer_forward writing `out` (not the buffer's) with the RMS norm, as
    between stacked layers, against the staged calls doing the same."""
    cfg = get_config("decode_fine", num_experts=40, hidden=512, ffn=256, shared_ffn=256)
    mats, experts = quantized_experts(cfg)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    x = G.activations(cfg, tokens=16, batch=5)
    ref = O.moe_layer(x, wr, b, experts, cfg.top_k, shared=shared)
    layer = make_gpu_layer(cfg, mats, wr, b, shared)
    buf = layer.alloc(16)
    o1 = torch.empty((16, cfg.hidden), dtype=torch.float16, device=buf.out.device)
    o2 = torch.empty_like(o1)
    xd = to_dev(x)
    layer.forward(xd, buf, rmsnorm=True, eps=cfg.rms_eps, out=o1)
    layer.forward_staged(xd, buf, rmsnorm=True, eps=cfg.rms_eps, out=o2)
    torch.cuda.synchronize()
    assert _np(o1).tobytes() == _np(o2).tobytes()
    ref = check_selection(ref, buf, 16, x, wr, b, experts, cfg, shared)
    tol_check(_np(o1), O.rmsnorm(ref["out"], cfg.rms_eps), "out")


@pytest.mark.parametrize("E,k", [(1, 1), (32, 1), (16, 4), (8, 8)])
def test_small_top_k_and_single_expert(E, k):
    """Top-1 (one expert per token, one-expert layers) and top-k = E."""
    cfg = get_config("decode_fine", num_experts=E, hidden=512, ffn=256, top_k=k,
                     shared_ffn=128)
    run_layer_case(cfg, 11, batch=E + k)


@pytest.mark.parametrize("T", [8, 150])
def test_layer_with_renormalised_weights(T):
    """moe_layer_forward with MOE_RENORM against the oracle layer whose
    combine divides each token's k weights by their sum."""
    cfg = get_config("decode_fine", num_experts=32, hidden=512, ffn=256, top_k=4,
                     shared_ffn=128)
    mats, experts = quantized_experts(cfg)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    x = G.activations(cfg, tokens=T, batch=3)
    ref = O.moe_layer(x, wr, b, experts, cfg.top_k, shared=shared)
    layer = make_gpu_layer(cfg, mats, wr, b, shared)
    buf = layer.alloc(T)
    out = _np(layer.forward(to_dev(x), buf, renorm=True))
    torch.cuda.synchronize()
    ref = check_selection(ref, buf, T, x, wr, b, experts, cfg, shared)
    out_ref = O.combine(ref["y_perm"], ref["ys"], ref["inv_pos"], ref["w"], T, cfg.top_k,
                        renorm=True)
    tol_check(out, out_ref, "renormalised out")


@pytest.mark.parametrize("T", [8, 150])
def test_layer_with_8bit_shared_expert(T):
    """A whole layer whose shared expert is 8-bit g128 (one-launch router at
    8 tokens, separate launches at 150), against the oracle layer whose
    shared expert uses the same dequantized 8-bit weights."""
    from gpu_util import shared_w8
    cfg = get_config("decode_fine", num_experts=32, hidden=512, ffn=256, top_k=4,
                     shared_ffn=256)
    mats, experts = quantized_experts(cfg)
    wr, b = G.router(cfg)
    stored8, deq = shared_w8(G.shared_expert(cfg))
    x = G.activations(cfg, tokens=T, batch=11)
    ref = oracle_layer(x, wr, b, experts, cfg, deq)
    layer = make_gpu_layer(cfg, mats, wr, b, None, w8=stored8)
    buf = layer.alloc(T)
    out = _np(layer.forward(to_dev(x), buf))
    torch.cuda.synchronize()
    tol_check(_np(buf.y_shared), ref["ys"], "8-bit shared expert")
    ref = check_selection(ref, buf, T, x, wr, b, experts, cfg, deq)
    tol_check(out, ref["out"], "layer out")


@pytest.mark.parametrize("T", [5, 2])
def test_largest_hidden_size(T):
    """hidden = 65536, the largest the ABI accepts: the one-launch router with
    its maximum of 16 K parts, gate/up rows of 128 KB streamed from memory
    (too large to stage in LDS), 4096 down-projection row tiles, and the
    combine over rows wider than one block (without the norm, and with it,
    the two-pass kernel for rows over 8192 columns); at 2 tokens the gate/up
    and shared items split their 512 quantization groups over 8 blocks.
    Expert weights are drawn as codes (the quantizer is pinned elsewhere)."""
    cfg = get_config("decode_fine", num_experts=3, hidden=65536, ffn=128, top_k=2,
                     shared_ffn=128)
    mats, experts = coded_experts(cfg)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    x = G.activations(cfg, tokens=T, batch=1)
    ref = O.moe_layer(x, wr, b, experts, cfg.top_k, shared=shared)
    layer = make_gpu_layer(cfg, mats, wr, b, shared)
    buf = layer.alloc(T)
    for rmsnorm in (False, True):
        out = _np(layer.forward(to_dev(x), buf, rmsnorm=rmsnorm, eps=cfg.rms_eps))
        torch.cuda.synchronize()
        r = check_selection(ref, buf, T, x, wr, b, experts, cfg, shared)
        want = O.rmsnorm(r["out"], cfg.rms_eps) if rmsnorm else r["out"]
        tol_check(out, want, f"H = 65536, norm {rmsnorm}")


def test_largest_ffn_size():
    """ffn = 262144, the largest the ABI accepts: 4096 gate/up row tiles per
    segment tile and a down projection whose K is 2048 blocks of 128."""
    cfg = get_config("tiny", num_experts=2, hidden=128, ffn=262144, top_k=1)
    mats, experts = coded_experts(cfg)
    wr, b = G.router(cfg)
    x = G.activations(cfg, tokens=3, batch=2)
    ref = O.moe_layer(x, wr, b, experts, cfg.top_k)
    layer = make_gpu_layer(cfg, mats, wr, b, None)
    buf = layer.alloc(3)
    out = _np(layer.forward(to_dev(x), buf))
    torch.cuda.synchronize()
    ref = check_selection(ref, buf, 3, x, wr, b, experts, cfg, None)
    tol_check(out, ref["out"], "F = 262144")


@pytest.mark.parametrize("T,gs", [(1, 128), (2, 128), (4, 128), (3, 64), (4, 256)])
def test_split_ffn_on_a_wide_layer(T, gs):
    """Batches of up to 4 tokens on a layer of hidden 16384: each gate/up item
    (64 rows of gate and of up, about 1 MB of codes) and each shared-expert
    item (1 MB of fp16) is split in K over up to 8 blocks, the down items stay
    whole.  At one token the token row (32 KB) is staged in LDS; from two
    tokens on the split blocks read their rows from memory.  With the
    permuted rows materialised (x_perm) the layer gives the same bits.
    Expert weights are drawn as codes."""
    cfg = get_config("decode_fine", num_experts=4, hidden=16384, ffn=256, top_k=2,
                     shared_ffn=256, group_size=gs)
    mats, experts = coded_experts(cfg)
    wr, b = G.router(cfg)
    shared = G.shared_expert(cfg)
    x = G.activations(cfg, tokens=T, batch=T)
    ref = oracle_layer(x, wr, b, experts, cfg, shared)
    layer = make_gpu_layer(cfg, mats, wr, b, shared)
    buf = layer.alloc(T)
    first = None
    for call in range(3):          # the tickets reset: later calls repeat the first bitwise
        out = _np(layer.forward(to_dev(x), buf))
        torch.cuda.synchronize()
        if first is None:
            first = out
            ref = check_selection(ref, buf, T, x, wr, b, experts, cfg, shared)
            tol_check(out, ref["out"], f"H = 16384, T = {T}, group {gs}")
        else:
            assert out.tobytes() == first.tobytes(), f"call {call}"
    out = _np(layer.forward(to_dev(x), buf, gather=True))
    torch.cuda.synchronize()
    assert out.tobytes() == first.tobytes(), "rows from x_perm"
