"""Stage-by-stage parity of the HIP kernels against the oracle (teacher-forced:
each C entry point is fed the oracle's inputs for that stage, so an upstream
near tie cannot cascade)."""
import numpy as np
import pytest
import torch

import oracle as O
from workloads import get_config
from workloads import gen as G

from gpu_util import (gpu, require_gpu, to_dev, tol_check, quantized_experts, make_gpu_layer,
                      route_compare, dev, shared_w8)

pytestmark = gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _np(t):
    return t.detach().cpu().numpy()


# ---------------------------------------------------------------- quantizer / dequant
@pytest.mark.parametrize("shape,gs", [((512, 256), 128), ((64, 4096), 128), ((48, 1024), 128),
                                      ((64, 4096), 64), ((48, 384), 64), ((32, 1024), 256),
                                      ((512, 256), 256)])
def test_quantize_bitexact(shape, gs):
    from w4_group_quantized_amd import quantize_fp16
    g = np.random.default_rng(shape[0] + gs)
    w = (g.standard_normal(shape, dtype=np.float32) * 0.02).astype(np.float16)
    w[3, :gs] = 0                                     # all-zero group
    w[5, shape[1] - gs:] = np.float16(1e-7)           # subnormal-range group
    w[6, :] = -w[6, :]
    q_ref, s_ref = O.group_quantize(w, gs)
    q, s = quantize_fp16(to_dev(w), gs)
    torch.cuda.synchronize()
    assert tuple(s.shape) == (shape[0], shape[1] // gs)
    np.testing.assert_array_equal(_np(s).view(np.uint16), O.pack_scales(s_ref).view(np.uint16))
    np.testing.assert_array_equal(_np(q), O.pack_w4(q_ref))


def test_quantize_golden_fixture():
    import json, os
    from w4_group_quantized_amd import quantize_fp16
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quantize_example.json")))
    w = np.zeros((16, fx["shape"][1]), dtype=np.float16)     # fixture row + 15 zero rows
    for c, v in fx["weights_nonzero"].items():
        w[0, int(c)] = v
    q, s = quantize_fp16(to_dev(w))
    torch.cuda.synchronize()
    assert [float(x) for x in O.unpack_scales(_np(s))[0]] == fx["expected_scales"]
    codes = O.unpack_w4(_np(q))[:1]
    exp = np.zeros(fx["shape"], dtype=np.int8)
    for c, v in fx["expected_codes_nonzero"].items():
        exp[0, int(c)] = v
    np.testing.assert_array_equal(codes, exp)


@pytest.mark.parametrize("shape", [(16, 128), (64, 4096), (48, 1024)])
def test_quantize_w8_bitexact(shape):
    """8-bit shared-expert codes and scales against the oracle, byte for byte."""
    from w4_group_quantized_amd import quantize_w8
    g = np.random.default_rng(shape[1])
    w = (g.standard_normal(shape, dtype=np.float32) * 0.02).astype(np.float16)
    w[3 % shape[0], :128] = 0
    w[5 % shape[0], -128:] = np.float16(3e-6)
    w[6 % shape[0], :] = -w[6 % shape[0], :]
    q_ref, s_ref = O.group_quantize(w, 128, bits=8)
    q, s = quantize_w8(to_dev(w))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(s).view(np.uint16), O.pack_scales(s_ref).view(np.uint16))
    np.testing.assert_array_equal(_np(q), O.pack_w8(q_ref))


@pytest.mark.parametrize("shape,gs", [((16, 128), 128), ((48, 1024), 64), ((64, 4096), 256),
                                      ((32, 512), 128)])
def test_pack_plain_codes_bitexact(shape, gs):
    """moe_w4_pack: plain row-major two's-complement codes (every byte value)
    and row-major scales -> the packed format, byte for byte what the oracle
    packs from the same codes."""
    from w4_group_quantized_amd import pack_plain
    g = np.random.default_rng(shape[1] + gs)
    plain = g.integers(0, 256, size=(shape[0], shape[1] // 2), dtype=np.uint8)
    plain.reshape(-1)[:256] = np.arange(256, dtype=np.uint8)      # every byte value
    s = g.uniform(1e-4, 5e-2, size=(shape[0], shape[1] // gs)).astype(np.float16)
    q, st = pack_plain(to_dev(plain), to_dev(s), gs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(q), O.pack_w4(O.unpack_plain_w4(plain)))
    np.testing.assert_array_equal(_np(st).view(np.uint16), O.pack_scales(s).view(np.uint16))


@pytest.mark.parametrize("gs", [64, 128, 256])
def test_dequant_bitexact_all_codes(gs):
    from w4_group_quantized_amd import dequantize
    g = np.random.default_rng(11)
    packed = g.integers(0, 256, size=(96, 384), dtype=np.uint8)    # every code, including -8
    packed[0, :256] = np.arange(256, dtype=np.uint8)
    s = (g.uniform(1e-4, 5e-2, size=(96, 768 // gs))).astype(np.float16)
    s[1, 2] = 0
    out = dequantize(to_dev(packed), to_dev(s))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(out).astype(np.float64), O.dequant(packed, s, gs))


# ---------------------------------------------------------------- router
ROUTE_CASES = [
    ("tiny", {}, 16),
    ("tiny", {}, 5),
    ("decode_fine", {}, 8),
    ("decode_fine", {}, 37),
    ("decode_coarse", {}, 16),
    ("prefill", {}, 300),
    ("decode_fine", {}, 333),      # 32-token x 128-expert tiles: 3 expert tiles, last one partial
    ("tiny", {}, 257),             # same tiles with 8 experts and a ragged token tail
    ("tiny", {"num_experts": 1024, "top_k": 32, "hidden": 512}, 6),   # largest E and k
    ("tiny", {"num_experts": 1000, "top_k": 7}, 300),                 # wide tiles, E % 128 != 0
]


@pytest.mark.parametrize("name,over,T", ROUTE_CASES)
def test_route(name, over, T):
    cfg = get_config(name, **over)
    wr, b = G.router(cfg)
    x = G.activations(cfg, tokens=T, batch=7)
    idx_ref, w_ref, l_ref = O.route(x, wr, b, cfg.top_k)
    layer = _router_only_layer(cfg, wr, b)
    buf = layer.alloc(T)
    layer.route(to_dev(x), buf, T)
    torch.cuda.synchronize()
    idx = _np(buf.topk_idx)
    if route_compare(idx, l_ref, cfg.top_k).any():   # weights of the GPU's selection
        w_ref = O.route(x, wr, b, cfg.top_k, idx=idx)[1]
    tol_check(_np(buf.topk_w), w_ref, "topk_w", rel=1e-5, abs_=1e-7)


def _router_only_layer(cfg, wr, b):
    from w4_group_quantized_amd import W4MoELayer
    z8 = to_dev(np.zeros((1, 1, 16), np.uint8))
    z16 = to_dev(np.zeros((1, 1, 8), np.float16))
    layer = W4MoELayer(cfg.top_k, to_dev(wr), to_dev(b) if b is not None else None,
                       z8, z16, z8, z16, z8, z16, group_size=cfg.group_size)
    layer.desc.ffn = cfg.ffn
    return layer


def test_route_duplicate_rows_lower_index_wins():
    cfg = get_config("decode_fine")
    wr, b = G.router(cfg)
    wr = wr.copy()
    b = b.copy()
    for lo, hi in ((3, 200), (17, 18), (0, 287)):
        wr[hi] = wr[lo]
        b[hi] = b[lo] = 3.0                          # make the pair win
    x = G.activations(cfg, tokens=24, batch=3)
    idx_ref, _, l_ref = O.route(x, wr, b, cfg.top_k)
    layer = _router_only_layer(cfg, wr, b)
    buf = layer.alloc(24)
    layer.route(to_dev(x), buf, 24)
    torch.cuda.synchronize()
    idx = _np(buf.topk_idx)
    np.testing.assert_array_equal(idx, idx_ref)      # exact ties: no near-tie excuse
    for lo, hi in ((3, 200), (17, 18), (0, 287)):
        for row in idx.tolist():
            if hi in row:
                assert lo in row and row.index(lo) < row.index(hi)


def test_route_nonfinite_inputs_give_valid_indices():
    cfg = get_config("tiny")
    wr, _ = G.router(cfg)
    x = G.activations(cfg, tokens=4).copy()
    x[1, 7] = np.float16(np.nan)
    x[2, 3] = np.float16(np.inf)
    layer = _router_only_layer(cfg, wr, None)
    buf = layer.alloc(4)
    layer.route(to_dev(x), buf, 4)
    torch.cuda.synchronize()
    idx = _np(buf.topk_idx)
    assert ((idx >= 0) & (idx < cfg.num_experts)).all()
    assert all(len(set(r)) == cfg.top_k for r in idx.tolist())
    w = _np(buf.topk_w)
    assert np.isfinite(w[[0, 3]]).all() and np.isnan(w[1]).all()


# ---------------------------------------------------------------- permutation
PERM_CASES = [
    (16, 2, 8, "random"),
    (8, 8, 288, "random"),
    (100, 8, 128, "random"),       # 800 entries: several chunks, ragged tail
    (1, 4, 16, "random"),
    (50, 1, 6, "one_expert"),
    (7, 5, 5, "k_eq_E"),
    (1000, 4, 1024, "random"),
    (8192, 8, 128, "random"),      # prefill size: 256 chunks split over 8 scan threads per expert
    (5000, 3, 3, "random"),        # 256 scan threads per expert
    (600, 1, 1, "random"),        # a single expert
]


@pytest.mark.parametrize("T,k,E,kind", PERM_CASES)
def test_permute_bitexact(T, k, E, kind):
    g = np.random.default_rng(T * 31 + k)
    if kind == "one_expert":
        idx = np.full((T, k), 3, dtype=np.int32)
    elif kind == "k_eq_E":
        idx = np.stack([g.permutation(E) for _ in range(T)]).astype(np.int32)
    else:
        idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    H = 256
    x = (g.standard_normal((T, H)) ).astype(np.float16)
    off, perm_src, inv_pos = O.permute(idx, E)
    xp_ref = O.gather_rows(x, perm_src, k)
    cfg = get_config("tiny", num_experts=E, top_k=k, hidden=H)
    wr = np.zeros((E, H), np.float16)
    layer = _router_only_layer(cfg, wr, None)
    buf = layer.alloc(T)
    buf.topk_idx.copy_(to_dev(idx))
    layer.permute(to_dev(x), buf, T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(buf.offsets), off)
    np.testing.assert_array_equal(_np(buf.perm_src), perm_src)
    np.testing.assert_array_equal(_np(buf.inv_pos), inv_pos)
    assert _np(buf.x_perm).tobytes() == xp_ref.tobytes()


@pytest.mark.parametrize("name,over,T", [("tiny", {}, 16), ("decode_fine", {}, 8),
                                         ("decode_fine", {}, 16), ("decode_fine", {}, 64),
                                         ("decode_coarse", {}, 16), ("decode_fine", {}, 65),
                                         ("prefill", {"tokens": 40}, 40),
                                         ("tiny", {"num_experts": 1024, "top_k": 32,
                                                   "hidden": 512}, 8)])   # T*E at the LDS limit
def test_route_permute_fused(name, over, T):
    """moe_route_permute (one launch for T <= 64) against the oracle: indices
    exact away from near ties; offsets/perm_src/inv_pos exact when the indices
    agree; called twice to check that the completion counter is reset."""
    cfg = get_config(name, **over)
    wr, b = G.router(cfg)
    layer = _router_only_layer(cfg, wr, b)
    buf = layer.alloc(T)
    for rep in range(2):
        x = G.activations(cfg, tokens=T, batch=20 + rep)
        idx_ref, w_ref, l_ref = O.route(x, wr, b, cfg.top_k)
        layer.route_permute(to_dev(x), buf, T, gather=True)
        torch.cuda.synchronize()
        idx = _np(buf.topk_idx)
        if route_compare(idx, l_ref, cfg.top_k).any():   # weights of the GPU's selection
            w_ref = O.route(x, wr, b, cfg.top_k, idx=idx)[1]
        tol_check(_np(buf.topk_w), w_ref, "topk_w", rel=1e-5, abs_=1e-7)
        # the permutation must be the exact permutation of the GPU's own indices
        off, perm_src, inv_pos = O.permute(idx, cfg.num_experts)
        np.testing.assert_array_equal(_np(buf.offsets), off)
        np.testing.assert_array_equal(_np(buf.perm_src), perm_src)
        np.testing.assert_array_equal(_np(buf.inv_pos), inv_pos)
        assert _np(buf.x_perm).tobytes() == O.gather_rows(x, perm_src, cfg.top_k).tobytes()


@pytest.mark.parametrize("nper", range(1, 17))
def test_topk_every_lane_count(nper):
    """Both top-k kernels (moe_route's and the one-launch moe_route_permute's)
    exist once per number of logits per lane, ceil(E / 64) = 1 .. 16: an
    expert count with a ragged last 64 for each, against the oracle."""
    E = 64 * nper - (13 * nper) % 64
    cfg = get_config("tiny", num_experts=E, top_k=min(8 + nper, E), hidden=256)
    wr, b = G.router(cfg)
    layer = _router_only_layer(cfg, wr, b)
    for T, fused in ((5, False), (6, True)):
        x = G.activations(cfg, tokens=T, batch=40 + nper)
        idx_ref, w_ref, l_ref = O.route(x, wr, b, cfg.top_k)
        buf = layer.alloc(T)
        if fused:
            layer.route_permute(to_dev(x), buf, T, gather=True)
        else:
            layer.route(to_dev(x), buf, T)
        torch.cuda.synchronize()
        idx = _np(buf.topk_idx)
        if route_compare(idx, l_ref, cfg.top_k).any():   # weights of the GPU's selection
            w_ref = O.route(x, wr, b, cfg.top_k, idx=idx)[1]
        tol_check(_np(buf.topk_w), w_ref, "topk_w", rel=1e-5, abs_=1e-7)
        if fused:
            off, perm_src, inv_pos = O.permute(idx, E)
            np.testing.assert_array_equal(_np(buf.offsets), off)
            np.testing.assert_array_equal(_np(buf.perm_src), perm_src)
            np.testing.assert_array_equal(_np(buf.inv_pos), inv_pos)


# ---------------------------------------------------------------- FFN
FFN_CASES = [
    ("tiny", {}, 16, 0, False),
    ("tiny", {"num_experts": 4, "top_k": 4}, 21, 0, False),             # >16 rows per segment
    ("tiny", {"num_experts": 12, "hidden": 512, "ffn": 384, "top_k": 3}, 9, 256, False),
    ("tiny", {"num_experts": 6, "hidden": 384, "ffn": 256, "top_k": 2}, 70, 128, False),
    # several rows per expert on average (the wider tile shapes); 16-row tiles
    # of 4 KB rows (64 KB: streamed from memory) next to 4-row ones (staged)
    ("tiny", {"num_experts": 4, "hidden": 2048, "ffn": 512, "top_k": 2}, 40, 256, False),
    # under two rows per expert on average, but every token also picks expert
    # 0: one 7-row tile of 8 KB rows (56 KB: streamed) among 1-row tiles
    ("tiny", {"num_experts": 8, "hidden": 4096, "ffn": 128, "top_k": 2}, 7, 128, True),
    # group sizes 64 and 256: one scale per 64 columns (folded into the
    # unpacked weights) and one per 256 (two K blocks per scale), on the
    # narrow and the wide tile shapes
    ("tiny", {"num_experts": 12, "hidden": 512, "ffn": 384, "top_k": 3, "group_size": 64}, 9,
     256, False),
    ("tiny", {"num_experts": 4, "hidden": 2048, "ffn": 512, "top_k": 2, "group_size": 64}, 40,
     256, False),
    ("tiny", {"num_experts": 12, "hidden": 512, "ffn": 256, "top_k": 3, "group_size": 256}, 9,
     256, False),
    ("tiny", {"num_experts": 4, "hidden": 2048, "ffn": 512, "top_k": 2, "group_size": 256}, 40,
     256, False),
    ("tiny", {"num_experts": 8, "hidden": 4096, "ffn": 256, "top_k": 2, "group_size": 64}, 7,
     128, True),
]


@pytest.mark.parametrize("use_x_perm", [False, True])
@pytest.mark.parametrize("name,over,T,Fs,skew", FFN_CASES)
def test_ffn_teacher_forced(name, over, T, Fs, skew, use_x_perm):
    run_ffn_case(name, over, T, Fs, skew, use_x_perm)


@pytest.mark.parametrize("over,T", [({"num_experts": 12, "hidden": 512, "ffn": 384, "top_k": 3}, 9),
                                    ({"num_experts": 4, "hidden": 2048, "ffn": 512, "top_k": 2}, 40),
                                    ({"num_experts": 2, "hidden": 256, "ffn": 256, "top_k": 2}, 70)])
def test_ffn_shared_w8(over, T):
    """The shared expert in 8 bits (g128) on the narrow and wide decode tile
    shapes and in prefill mode (70 tokens over 2 experts), 3 token tiles at
    most, K of 2 to 16 blocks split over 4 waves."""
    run_ffn_case("tiny", over, T, 384, False, False, w8=True)


def run_ffn_case(name, over, T, Fs, skew, use_x_perm, w8=False):
    cfg = get_config(name, shared_ffn=Fs, **over)
    mats, experts = quantized_experts(cfg)
    wr, b = G.router(cfg)
    x = G.activations(cfg, tokens=T, batch=5)
    shared = G.shared_expert(cfg) if Fs else None
    stored8 = None
    if w8:
        stored8, shared = shared_w8(shared)     # oracle: the dequantized 8-bit weights
    if skew:                     # token t -> experts 0 and 1 + t % (E - 1)
        idx = np.stack([np.zeros(T, np.int32), 1 + np.arange(T, dtype=np.int32) %
                        (cfg.num_experts - 1)], axis=1)
    else:
        idx, w, l = O.route(x, wr, b, cfg.top_k)
    off, perm_src, inv_pos = O.permute(idx, cfg.num_experts)
    x_perm = O.gather_rows(x, perm_src, cfg.top_k)
    layer = make_gpu_layer(cfg, mats, wr, b, None if w8 else shared, w8=stored8)
    buf = layer.alloc(T)
    buf.offsets.copy_(to_dev(off))
    if use_x_perm:
        buf.x_perm.copy_(to_dev(x_perm))
        buf.perm_src.fill_(-1)                    # must not be read
    else:
        buf.perm_src.copy_(to_dev(perm_src))
        buf.x_perm.fill_(float("nan"))            # must not be read
    layer.ffn(to_dev(x), buf, T, use_x_perm=use_x_perm)
    torch.cuda.synchronize()
    y_perm = _np(buf.y_perm)
    for e in range(cfg.num_experts):
        a, bnd = int(off[e]), int(off[e + 1])
        if bnd > a:
            ref = O.expert_ffn_w4(x_perm[a:bnd], *experts[e], group=cfg.group_size)
            tol_check(y_perm[a:bnd], ref, f"expert {e}")
    if Fs:
        tol_check(_np(buf.y_shared), O.swiglu_ffn(x, *shared), "shared")


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("T,k,H,with_shared", [(16, 2, 256, False), (9, 8, 4096, True),
                                               (3, 32, 384, True), (5, 8, 6144, True),
                                               (4, 3, 12416, False), (2, 4, 20480, True)])
def test_combine(T, k, H, with_shared, rms, renorm):
    g = np.random.default_rng(T + k)
    N = T * k
    y_perm = (g.standard_normal((N, H)) * 0.3).astype(np.float16)
    ys = (g.standard_normal((T, H)) * 0.3).astype(np.float16) if with_shared else None
    inv = g.permutation(N).astype(np.int32)
    w = g.uniform(0, 0.3, size=(T, k)).astype(np.float32)
    ref = O.combine(y_perm, ys, inv, w, T, k, renorm=renorm)
    if rms:
        ref = O.rmsnorm(ref, 1e-6)
    E = max(k, 8)
    cfg = get_config("tiny", num_experts=E, top_k=k, hidden=H, shared_ffn=128 if with_shared else 0)
    layer = _router_only_layer(cfg, np.zeros((E, H), np.float16), None)
    if with_shared:
        layer.Fs = 128
        layer.desc.shared_ffn = 128
    buf = layer.alloc(T)
    buf.y_perm.copy_(to_dev(y_perm))
    if with_shared:
        buf.y_shared.copy_(to_dev(ys))
    buf.inv_pos.copy_(to_dev(inv))
    buf.topk_w.copy_(to_dev(w))
    layer.combine(buf, T, rmsnorm=rms, renorm=renorm)
    torch.cuda.synchronize()
    tol_check(_np(buf.out), ref, "combine")


def test_combine_rows_past_4_gib():
    """Hidden 65536 and 32784 tokens: the shared expert's rows and the output
    rows of the last tokens start more than 2^32 bytes into their buffers
    (t * H * 2 >= 2^32 from t = 32768); the combine must still read each
    token's own shared row.  Checked on the first and the last 16 tokens."""
    from types import SimpleNamespace
    T, k, H = 32784, 1, 65536
    cfg = get_config("tiny", num_experts=8, top_k=k, hidden=H, shared_ffn=128)
    layer = _router_only_layer(cfg, np.zeros((8, H), np.float16), None)
    layer.Fs = 128
    layer.desc.shared_ffn = 128
    g = torch.Generator(device=dev())
    g.manual_seed(1234)
    f16 = torch.float16
    bufs = SimpleNamespace(
        y_perm=(torch.randn((T * k, H), generator=g, device=dev()) * 0.3).to(f16),
        y_shared=(torch.randn((T, H), generator=g, device=dev()) * 0.3).to(f16),
        inv_pos=torch.randperm(T * k, generator=g, device=dev()).to(torch.int32),
        topk_w=torch.rand((T, k), generator=g, device=dev()) * 0.3,
        out=torch.empty((T, H), dtype=f16, device=dev()))
    layer.combine(bufs, T)
    torch.cuda.synchronize()
    toks = np.r_[0:16, T - 16:T]
    inv = _np(bufs.inv_pos).astype(np.int64)
    w = _np(bufs.topk_w).astype(np.float64)
    for t in toks:
        ys = _np(bufs.y_shared[t]).astype(np.float64)
        yp = _np(bufs.y_perm[inv[t]]).astype(np.float64)
        ref = O.combine(yp[None], ys[None], np.zeros(1, np.int64), w[t:t + 1], 1, 1)[0]
        tol_check(_np(bufs.out[t]), ref, f"token {t}")
    del bufs


# ---------------------------------------------------------------- exact-arithmetic probe
def _probe_codes(rng, rows, cols, kind):
    """Integer codes for the exact probe: 'gate' rows have 20 leading ones
    plus sparse ones (every gate pre-activation is an integer >= 20 for
    activations in {1, 2}); 'up' and 'down' are sparse -1/0/1."""
    if kind == "gate":
        q = (rng.random((rows, cols)) < 0.05).astype(np.int8)
        q[:, :20] = 1
    else:
        q = rng.choice(np.array([-1, 0, 1], np.int8), size=(rows, cols), p=[0.02, 0.96, 0.02])
    return q


@pytest.mark.parametrize("E,k,T,shared", [(6, 2, 9, True),      # narrow decode tiles
                                          (3, 2, 40, False),    # wide decode tiles
                                          (2, 2, 80, True)])    # prefill MFMA kernel
def test_ffn_exact_integer_probe(E, k, T, shared):
    """Activations in {1, 2}, integer codes and unit scales keep every gate and
    up dot product, h = silu(g) * u (silu(g) = g exactly in fp32 for g >= 20)
    and the down projection integers below 2048, so fp32 accumulation and the
    fp16 outputs are exact: the GPU must return integers equal to the oracle
    up to the oracle's own float64 silu (relative 1e-8), far inside the usual
    bound."""
    H, F, Fs = 128, 128, 128 if shared else 0
    cfg = get_config("tiny", num_experts=E, hidden=H, ffn=F, top_k=k, shared_ffn=Fs)
    rng = np.random.default_rng(E * 100 + T)
    one = lambda rows, cols: np.ones((rows, cols // 128), np.float16)  # noqa: E731
    mats = {n: [] for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}
    experts = []
    for e in range(E):
        tup = []
        for name, (rows, cols) in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
            p, s = O.pack_w4(_probe_codes(rng, rows, cols, name)), O.pack_scales(one(rows, cols))
            mats[name + "_q"].append(p)
            mats[name + "_s"].append(s)
            tup += [p, s]
        experts.append(tuple(tup))
    mats = {n: np.stack(v) for n, v in mats.items()}
    sh = None
    if shared:
        sh = tuple(_probe_codes(rng, r, c, kind).astype(np.float16)
                   for kind, (r, c) in (("gate", (Fs, H)), ("up", (Fs, H)), ("down", (H, Fs))))
    x = rng.integers(1, 3, size=(T, H)).astype(np.float16)
    idx = np.stack([(np.arange(T) + j) % E for j in range(k)], axis=1).astype(np.int32)
    off, perm_src, inv_pos = O.permute(idx, E)
    x_perm = O.gather_rows(x, perm_src, k)
    wr = np.zeros((E, H), np.float16)
    layer = make_gpu_layer(cfg, mats, wr, None, sh)
    buf = layer.alloc(T)
    buf.offsets.copy_(to_dev(off))
    buf.perm_src.copy_(to_dev(perm_src))
    layer.ffn(to_dev(x), buf, T)
    torch.cuda.synchronize()
    y = _np(buf.y_perm).astype(np.float64)
    assert (y == np.rint(y)).all() and np.abs(y).max() < 2048
    for e in range(E):
        a, bnd = int(off[e]), int(off[e + 1])
        if bnd > a:
            ref = O.expert_ffn_w4(x_perm[a:bnd], *experts[e])
            assert np.abs(ref).max() > 10          # a non-trivial probe
            np.testing.assert_allclose(y[a:bnd], ref, rtol=1e-8, atol=1e-6)
    if shared:
        ys = _np(buf.y_shared).astype(np.float64)
        ref = O.swiglu_ffn(x, *sh)
        assert (ys == np.rint(ys)).all()
        np.testing.assert_allclose(ys, ref, rtol=1e-8, atol=1e-6)
