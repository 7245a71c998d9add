"""Pins of the float64 oracle against facts fixed outside it.

Each test checks the oracle against something it does not compute itself:
values derived by hand (tests/golden), exact rational arithmetic, brute force
on tiny inputs, closed forms and invariants.  None of these needs a GPU.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from workloads import get_config
from workloads import gen as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# every finite fp16 value, ascending, as exact Fractions (for brute force)
_F16_BITS = np.arange(0, 0x7C00, dtype=np.uint16)                 # +0 .. max finite
_F16_POS = _F16_BITS.view(np.float16).astype(np.float64)


def nearest_f16(v: Fraction) -> Fraction:
    """Round a rational to fp16 by searching all finite fp16 values
    (ties to the value with an even bit pattern)."""
    sign = -1 if v < 0 else 1
    a = abs(v)
    i = int(np.searchsorted(_F16_POS, float(a)))
    cands = set()
    for j in (i - 2, i - 1, i, i + 1):
        if 0 <= j < _F16_POS.size:
            cands.add(j)
    best = min(cands, key=lambda j: (abs(Fraction(_F16_POS[j]) - a), int(_F16_BITS[j]) & 1))
    return sign * Fraction(_F16_POS[best])


# ---------------------------------------------------------------- fp16 rounding
def test_rn16_matches_bruteforce_nearest():
    g = np.random.default_rng(1)
    vals = np.concatenate([
        g.standard_normal(300) * 0.02, g.standard_normal(300) * 7,
        # exact midpoints between neighbouring fp16 values (tie cases)
        (_F16_POS[1000:1100] + _F16_POS[1001:1101]) / 2,
        (_F16_POS[20000:20100] + _F16_POS[20001:20101]) / 2,
    ])
    got = O.rn16(vals)
    for v, r in zip(vals, got):
        assert Fraction(r) == nearest_f16(Fraction(v)), v


# ---------------------------------------------------------------- quantizer
def test_quantizer_golden_example():
    fx = json.load(open(os.path.join(GOLDEN, "quantize_example.json")))
    w = np.zeros(fx["shape"], dtype=np.float16)
    for c, v in fx["weights_nonzero"].items():
        w[0, int(c)] = v
        assert float(np.float16(v)) == v          # fixture values are exact fp16
    q, s = O.group_quantize(w, fx["group_size"])
    assert s.dtype == np.float16 and q.dtype == np.int8
    assert [float(x) for x in s[0]] == fx["expected_scales"]
    exp = np.zeros(fx["shape"], dtype=np.int8)
    for c, v in fx["expected_codes_nonzero"].items():
        exp[0, int(c)] = v
    np.testing.assert_array_equal(q, exp)


@pytest.mark.parametrize("group", [64, 128, 256])
def test_quantizer_exact_rational_bruteforce(group):
    """Recompute s and q for random fp16 weights with exact rational
    arithmetic and a brute-force fp16 rounding, independent of float64."""
    g = np.random.default_rng(2)
    w = (g.standard_normal((3, 512)) * 0.02).astype(np.float16)
    q, s = O.group_quantize(w, group)
    assert s.shape == (3, 512 // group)
    for n in range(w.shape[0]):
        for grp in range(512 // group):
            ws = [Fraction(float(v)) for v in w[n, grp * group:(grp + 1) * group]]
            m = max(abs(v) for v in ws)
            s_ref = nearest_f16(m / 7)
            assert Fraction(float(s[n, grp])) == s_ref
            for c, v in enumerate(ws):
                r = nearest_f16(v / s_ref)
                q_ref = max(-8, min(7, round(r)))          # round(): half to even
                assert int(q[n, grp * group + c]) == q_ref


@pytest.mark.parametrize("group", [64, 128, 256])
def test_quantizer_invariants(group):
    cfg = get_config("tiny")
    w = G.expert_master(cfg, 0, 3, G.GATE).astype(np.float16)       # [512, 256]
    w[5, 256 - group:256] = 0                                       # an all-zero group
    q, s = O.group_quantize(w, group)
    assert q.min() >= -7 and q.max() <= 7                           # -8 never produced
    qa = np.abs(q.astype(np.int32)).reshape(q.shape[0], -1, group).max(-1)
    nz = s.astype(np.float64) > 0
    assert (qa[nz] == 7).all()
    assert (qa[~nz] == 0).all() and not nz[5, -1]
    err = np.abs(w.astype(np.float64) - O.dequant(O.pack_w4(q), O.pack_scales(s), group))
    bound = (0.5 + 2.0 ** -9) * np.repeat(s.astype(np.float64), group, axis=1)
    assert (err <= bound).all()


def test_quantizer_refuses_ragged_in_features():
    with pytest.raises(ValueError):
        O.group_quantize(np.zeros((2, 200), dtype=np.float16))


# ---------------------------------------------------------------- packing / dequant
def test_pack_layout_exhaustive():
    """Every byte value at many storage offsets of a [32, 256] matrix, against
    the documented layout: offset(row n, chunk c, byte b) = (n//16)*16*128 +
    c*256 + (n%16)*16 + b; byte b holds, as (low, high) nibble, columns
    32c + 8*(b//4) + {0:(0,2), 1:(4,6), 2:(1,3), 3:(5,7)}[b%4]; value = nibble-8."""
    table = {0: (0, 2), 1: (4, 6), 2: (1, 3), 3: (5, 7)}
    rows, cols = 32, 256
    rng = np.random.default_rng(12)
    for v in range(256):
        n, c, b = int(rng.integers(rows)), int(rng.integers(cols // 32)), int(rng.integers(16))
        flat = np.zeros(rows * cols // 2, dtype=np.uint8)
        flat[(n // 16) * 16 * (cols // 2) + c * 256 + (n % 16) * 16 + b] = v
        q = O.unpack_w4(flat.reshape(rows, cols // 2))
        lo, hi = table[b % 4]
        base = 32 * c + 8 * (b // 4)
        expect = np.full((rows, cols), -8, dtype=np.int8)
        expect[n, base + lo] = (v & 15) - 8
        expect[n, base + hi] = (v >> 4) - 8
        np.testing.assert_array_equal(q, expect)
        np.testing.assert_array_equal(O.pack_w4(q).reshape(-1), flat)


def test_plain_int4_layout_hand_example():
    """Plain row-major storage: low nibble = even column, two's complement."""
    b = np.zeros((1, 4), np.uint8)
    b[0] = [0x8F, 0x07, 0x71, 0xF8]
    assert O.unpack_plain_w4(b).tolist() == [[-1, -8, 7, 0, 1, 7, -8, -1]]
    # every byte value: the two nibbles decode independently
    allb = np.arange(256, dtype=np.uint8).reshape(16, 16)
    q = O.unpack_plain_w4(allb).reshape(-1, 2)
    for v in range(256):
        lo, hi = v & 15, v >> 4
        assert q[v, 0] == (lo - 16 if lo >= 8 else lo) and q[v, 1] == (hi - 16 if hi >= 8 else hi)


def test_scale_layout():
    """offset(row n, group g) = (n//16)*16*G + g*16 + n%16."""
    rows, G = 32, 3
    s = (np.arange(rows * G, dtype=np.float64).reshape(rows, G) + 1).astype(np.float16)
    st = O.pack_scales(s).reshape(-1)
    for n in range(rows):
        for g in range(G):
            assert st[(n // 16) * 16 * G + g * 16 + n % 16] == s[n, g]
    np.testing.assert_array_equal(O.unpack_scales(O.pack_scales(s)), s)


@pytest.mark.parametrize("group", [64, 128, 256])
def test_dequant_exact(group):
    g = np.random.default_rng(3)
    q = g.integers(-8, 8, size=(16, 256)).astype(np.int8)
    s = (g.uniform(1e-3, 1e-2, size=(16, 256 // group))).astype(np.float16)
    W = O.dequant(O.pack_w4(q), O.pack_scales(s), group)
    for n in range(16):
        for c in range(0, 256, 7):
            assert Fraction(W[n, c]) == int(q[n, c]) * Fraction(float(s[n, c // group]))
    # q*s is exact in fp32 as well (4 + 11 significant bits)
    np.testing.assert_array_equal(W.astype(np.float32).astype(np.float64), W)


# ---------------------------------------------------------------- 8-bit shared expert
def test_w8_quantizer_exact_rational_bruteforce():
    """8-bit codes: s = RN16(max|w| / 127), q = clamp(RNE(RN16(w / s)), -128,
    127), recomputed with exact rationals and brute-force fp16 rounding."""
    g = np.random.default_rng(21)
    w = (g.standard_normal((2, 256)) * 0.02).astype(np.float16)
    q, s = O.group_quantize(w, 128, bits=8)
    for n in range(2):
        for grp in range(2):
            ws = [Fraction(float(v)) for v in w[n, grp * 128:(grp + 1) * 128]]
            s_ref = nearest_f16(max(abs(v) for v in ws) / 127)
            assert Fraction(float(s[n, grp])) == s_ref
            for c, v in enumerate(ws):
                q_ref = max(-128, min(127, round(nearest_f16(v / s_ref))))
                assert int(q[n, grp * 128 + c]) == q_ref


def test_w8_quantizer_invariants():
    cfg = get_config("tiny")
    w = G.expert_master(cfg, 0, 5, G.UP).astype(np.float16)          # [512, 256]
    w[7, :128] = 0
    q, s = O.group_quantize(w, 128, bits=8)
    assert q.min() >= -127 and q.max() <= 127                        # -128 never produced
    qa = np.abs(q.astype(np.int32)).reshape(q.shape[0], -1, 128).max(-1)
    nz = s.astype(np.float64) > 0
    assert (qa[nz] == 127).all() and (qa[~nz] == 0).all() and not nz[7, 0]
    err = np.abs(w.astype(np.float64) - O.dequant_w8(O.pack_w8(q), O.pack_scales(s)))
    # |w/s - RN16(w/s)| <= 2^-5 below 128, plus the final rounding to an integer
    bound = (0.5 + 2.0 ** -5) * np.repeat(s.astype(np.float64), 128, axis=1)
    assert (err <= bound).all()


def test_w8_pack_layout_every_byte():
    """Every byte value at random storage offsets of a [32, 256] matrix,
    against byte(n, c) = (n//16)*16*256 + (c//16)*256 + (n%16)*16 + c%16 and
    value = byte - 128."""
    rows, cols = 32, 256
    rng = np.random.default_rng(22)
    for v in range(256):
        n, c = int(rng.integers(rows)), int(rng.integers(cols))
        flat = np.full(rows * cols, 128, dtype=np.uint8)
        flat[(n // 16) * 16 * cols + (c // 16) * 256 + (n % 16) * 16 + c % 16] = v
        q = O.unpack_w8(flat.reshape(rows, cols))
        expect = np.zeros((rows, cols), dtype=np.int8)
        expect[n, c] = v - 128
        np.testing.assert_array_equal(q, expect)
        np.testing.assert_array_equal(O.pack_w8(q).reshape(-1), flat)


def test_w8_dequant_exact():
    g = np.random.default_rng(23)
    q = g.integers(-128, 128, size=(16, 256)).astype(np.int8)
    s = g.uniform(1e-4, 1e-3, size=(16, 2)).astype(np.float16)
    W = O.dequant_w8(O.pack_w8(q), O.pack_scales(s))
    for n in range(16):
        for c in range(0, 256, 5):
            assert Fraction(W[n, c]) == int(q[n, c]) * Fraction(float(s[n, c // 128]))
    # q*s needs at most 8 + 11 bits: exact in fp32
    np.testing.assert_array_equal(W.astype(np.float32).astype(np.float64), W)


# ---------------------------------------------------------------- router
def test_softmax_closed_form():
    E = 6
    l = np.log(np.arange(1, E + 1, dtype=np.float64))[None, :] + 3.0
    p = O.softmax(l)
    np.testing.assert_allclose(p[0], np.arange(1, E + 1) / (E * (E + 1) / 2), rtol=1e-15)


def test_router_logits_bruteforce():
    g = np.random.default_rng(4)
    x = g.standard_normal((3, 5)).astype(np.float16)
    wr = (g.standard_normal((4, 5)) * 0.1).astype(np.float16)
    b = g.standard_normal(4).astype(np.float32)
    l = O.router_logits(x, wr, b)
    for t in range(3):
        for e in range(4):
            ref = math.fsum(float(x[t, h]) * float(wr[e, h]) for h in range(5)) + float(b[e])
            assert abs(l[t, e] - ref) <= 1e-15 * (1 + abs(ref))


def test_topk_bruteforce_all_subsets():
    g = np.random.default_rng(5)
    E, k = 7, 3
    for _ in range(40):
        l = np.round(g.standard_normal((1, E)) * 2) / 2          # many exact ties
        idx = O.topk_order(l, k)[0].tolist()
        # brute force: the best subset under (-logit, index) lexicographic order
        best = min(itertools.permutations(range(E), k),
                   key=lambda c: [(-l[0, e], e) for e in c])
        assert idx == list(best)


def test_route_duplicate_rows_tie_lower_index_wins():
    cfg = get_config("tiny")
    x = G.activations(cfg)
    wr, _ = G.router(cfg)
    wr = wr.copy()
    wr[6] = wr[1]                                 # experts 1 and 6 tie exactly
    wr[1] = wr[1] * np.float16(4)                 # and make them win most tokens
    wr[6] = wr[1]
    idx, w, l = O.route(x, wr, None, 2)
    assert (l[:, 1] == l[:, 6]).all()
    for t in range(x.shape[0]):
        row = idx[t].tolist()
        if 6 in row:
            assert 1 in row and row.index(1) < row.index(6)
    np.testing.assert_allclose(O.softmax(l).sum(1), 1.0, rtol=1e-14)


def test_tie_excused_hand_cases():
    """The reported-tie rule on hand-built logits: which position differs and
    by how much decides, not whether some pair of the token is close."""
    l = np.array([
        [3.0, 1.0, 1.0 + 5e-7, -2.0],   # experts 2, 1 within 5e-7
        [3.0, 1.0, 1.0 + 5e-7, -2.0],
        [3.0, 1.0, 1.0 + 5e-7, -2.0],
        [3.0, 2.0, 2.0 - 4e-7, 0.0],    # 1, 2 close: the k-th and (k+1)-th
        [3.0, 2.0, 1.0, 0.0],
        [3.0, 3.0 - 2e-6, 1.0, 0.0],    # 2e-6 apart: beyond the gap
    ])
    other = np.array([
        [0, 2],   # the oracle's own order: no difference
        [0, 1],   # 1 for 2 at position 1, 5e-7 apart: excused
        [2, 0],   # 2 at position 0 where the oracle has 0: 2 apart, failed
        [0, 2],   # boundary swap with the (k+1)-th expert, 4e-7 apart: excused
        [0, 2],   # 2 for 1: 1 apart, failed
        [1, 0],   # a swap 2e-6 apart: failed
    ])
    differs, excused = O.tie_excused(other, l)
    assert differs.tolist() == [False, True, True, True, True, True]
    assert excused.tolist() == [False, True, False, True, False, False]
    # a close pair elsewhere in the list does not excuse a wrong expert at
    # another position (the close pair is 2, 1; the mistake is 3 for 2)
    l2 = np.array([[5.0, 4.0, 4.0 + 1e-7, 1.0, 0.0]])
    d, e = O.tie_excused(np.array([[0, 2, 3]]), l2)
    assert d.tolist() == [True] and e.tolist() == [False]
    # a repeated or out-of-range expert is never excused
    l3 = np.array([[1.0, 1.0, 0.0]])
    assert O.tie_excused(np.array([[1, 1]]), l3)[1].tolist() == [False]
    assert O.tie_excused(np.array([[1, 7]]), l3)[1].tolist() == [False]


def test_route_on_a_given_selection():
    """route(..., idx=sel) returns the softmax probabilities of the given
    experts, computed here by explicit exp sums; with the oracle's own
    selection it equals the unforced route."""
    cfg = get_config("tiny", num_experts=6, hidden=128, top_k=3)
    wr, b = G.router(cfg)
    x = G.activations(cfg, tokens=4, batch=2)
    idx0, w0, l0 = O.route(x, wr, b, 3)
    idx1, w1, _ = O.route(x, wr, b, 3, idx=idx0)
    assert (idx1 == idx0).all() and np.array_equal(w1, w0)
    sel = np.array([[5, 0, 2], [1, 2, 3], [4, 3, 0], [0, 1, 5]])
    idx2, w2, l2 = O.route(x, wr, b, 3, idx=sel)
    assert (idx2 == sel).all()
    for t in range(4):
        den = math.fsum(math.exp(v) for v in l2[t])
        for j in range(3):
            assert abs(w2[t, j] - math.exp(l2[t, sel[t, j]]) / den) <= 1e-15
    with pytest.raises(ValueError):
        O.route(x, wr, b, 3, idx=np.array([[0, 0, 1]] * 4))
    with pytest.raises(ValueError):
        O.route(x, wr, b, 3, idx=np.array([[0, 6, 1]] * 4))


# ---------------------------------------------------------------- permutation
def test_permute_bruteforce_definition():
    g = np.random.default_rng(6)
    T, k, E = 13, 3, 9
    idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[4] = [2, 0, 8]
    off, perm_src, inv_pos = O.permute(idx, E)
    flat = idx.reshape(-1).tolist()
    cnt = [flat.count(e) for e in range(E)]
    assert off.tolist() == [sum(cnt[:e]) for e in range(E + 1)]
    for f, e in enumerate(flat):
        r = off[e] + sum(1 for f2 in range(f) if flat[f2] == e)
        assert inv_pos[f] == r and perm_src[r] == f
    x = g.standard_normal((T, 16)).astype(np.float16)
    xp = O.gather_rows(x, perm_src, k)
    for f in range(T * k):
        assert xp[inv_pos[f]].tobytes() == x[f // k].tobytes()


def test_permute_all_to_one_expert_and_k_equals_E():
    idx = np.zeros((5, 1), dtype=np.int32) + 3
    off, perm_src, inv_pos = O.permute(idx, 6)
    assert off.tolist() == [0, 0, 0, 0, 5, 5, 5]
    assert perm_src.tolist() == [0, 1, 2, 3, 4]
    idx = np.array([[2, 0, 1], [1, 2, 0]], dtype=np.int32)
    off, perm_src, _ = O.permute(idx, 3)
    assert off.tolist() == [0, 2, 4, 6]
    assert perm_src.tolist() == [1, 5, 2, 3, 0, 4]


# ---------------------------------------------------------------- FFN / layer
def test_silu_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 40.0, -800.0])
    s = O.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(s[2] + 0.25 * math.log(3.0)) < 1e-15
    assert abs(s[3] - 40.0) < 1e-12
    assert s[4] == 0.0


def test_swiglu_small_loops():
    """Pure-Python loops over tiny matrices: catches a transposed operand."""
    g = np.random.default_rng(7)
    X = g.standard_normal((2, 3))
    Wg = g.standard_normal((4, 3))
    Wu = g.standard_normal((4, 3))
    Wd = g.standard_normal((3, 4))
    Y = O.swiglu_ffn(X, Wg, Wu, Wd)
    for t in range(2):
        h = []
        for f in range(4):
            gg = sum(X[t, c] * Wg[f, c] for c in range(3))
            uu = sum(X[t, c] * Wu[f, c] for c in range(3))
            h.append(gg / (1 + math.exp(-gg)) * uu)
        for o in range(3):
            ref = sum(h[f] * Wd[o, f] for f in range(4))
            assert abs(Y[t, o] - ref) < 1e-12


def _tiny_layer(cfg, layer=0):
    x = G.activations(cfg, layer=layer)
    wr, b = G.router(cfg, layer)
    experts = []
    for e in range(cfg.num_experts):
        mats = []
        for m in (G.GATE, G.UP, G.DOWN):
            q, s = O.group_quantize(G.expert_master(cfg, layer, e, m))
            mats += [O.pack_w4(q), O.pack_scales(s)]
        experts.append(tuple(mats))
    return x, wr, b, experts


def test_layer_equals_dense_all_experts_then_mask():
    cfg = get_config("tiny")
    x, wr, b, experts = _tiny_layer(cfg)
    res = O.moe_layer(x, wr, b, experts, cfg.top_k)
    p = O.softmax(O.router_logits(x, wr, b))
    dense = np.zeros((cfg.tokens, cfg.hidden))
    for e in range(cfg.num_experts):
        Ye = O.expert_ffn_w4(x, *experts[e])                     # every token, every expert
        mask = (res["idx"] == e).any(axis=1)
        dense += (p[:, e] * mask)[:, None] * Ye
    np.testing.assert_allclose(res["out"], dense, rtol=0, atol=1e-12 * np.abs(dense).max())


def test_layer_on_a_given_selection_equals_dense_then_mask():
    """The layer evaluated on a forced selection (the path used at a reported
    near tie): every expert on every token, masked by the given selection and
    weighted by its softmax probability."""
    cfg = get_config("tiny")
    x, wr, b, experts = _tiny_layer(cfg)
    g = np.random.default_rng(11)
    sel = np.stack([g.choice(cfg.num_experts, cfg.top_k, replace=False)
                    for _ in range(cfg.tokens)])
    res = O.moe_layer(x, wr, b, experts, cfg.top_k, idx=sel)
    p = O.softmax(O.router_logits(x, wr, b))
    dense = np.zeros((cfg.tokens, cfg.hidden))
    for e in range(cfg.num_experts):
        Ye = O.expert_ffn_w4(x, *experts[e])
        mask = (sel == e).any(axis=1)
        dense += (p[:, e] * mask)[:, None] * Ye
    np.testing.assert_allclose(res["out"], dense, rtol=0, atol=1e-12 * np.abs(dense).max())
    off, perm_src, _ = O.permute(sel, cfg.num_experts)
    assert (res["offsets"] == off).all() and (res["perm_src"] == perm_src).all()


def test_layer_special_cases():
    cfg = get_config("tiny", num_experts=1, top_k=1)
    x, wr, b, experts = _tiny_layer(cfg)
    res = O.moe_layer(x, wr, b, experts, 1)
    np.testing.assert_allclose(res["w"], 1.0, rtol=1e-15)      # softmax of one logit
    np.testing.assert_allclose(res["out"], O.expert_ffn_w4(x, *experts[0]), rtol=1e-13, atol=0)

    # k = E: a dense softmax mixture of all experts
    cfg = get_config("tiny", num_experts=3, top_k=3)
    x, wr, b, experts = _tiny_layer(cfg)
    res = O.moe_layer(x, wr, b, experts, 3)
    p = O.softmax(O.router_logits(x, wr, b))
    mix = sum(p[:, e:e + 1] * O.expert_ffn_w4(x, *experts[e]) for e in range(3))
    np.testing.assert_allclose(res["out"], mix, rtol=0, atol=1e-12 * np.abs(mix).max())

    # x = 0: silu(0) = 0, so every expert and the shared expert give 0
    cfg = get_config("tiny")
    _, wr, b, experts = _tiny_layer(cfg)
    z = np.zeros((4, cfg.hidden), dtype=np.float16)
    sh = tuple(G.normal16(np.random.default_rng(8), s, 0.02)
               for s in ((64, cfg.hidden), (64, cfg.hidden), (cfg.hidden, 64)))
    res = O.moe_layer(z, wr, b, experts, cfg.top_k, shared=sh)
    assert not res["out"].any()

    # identical experts: out = ys + (sum_j w_j) * FFN(x)
    x, wr, b, experts = _tiny_layer(cfg)
    same = [experts[0]] * cfg.num_experts
    res = O.moe_layer(x, wr, b, same, cfg.top_k, shared=sh)
    ref = O.swiglu_ffn(x, *sh) + res["w"].sum(1, keepdims=True) * O.expert_ffn_w4(x, *experts[0])
    np.testing.assert_allclose(res["out"], ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_combine_renormalised_weights():
    """With renorm the k weights act as a convex combination: identical
    expert rows come back unchanged, and scaling every weight of a token by a
    constant changes nothing; against loops that divide by the sum."""
    g = np.random.default_rng(19)
    T, k, H = 5, 3, 4
    ys = g.standard_normal((T, H))
    inv = g.permutation(T * k).astype(np.int32)
    w = g.uniform(0.01, 0.3, size=(T, k))
    v = g.standard_normal(H)
    same = np.tile(v, (T * k, 1))
    out = O.combine(same, ys, inv, w, T, k, renorm=True)
    np.testing.assert_allclose(out, ys + v[None, :], rtol=0, atol=1e-14)
    y_perm = g.standard_normal((T * k, H))
    a = O.combine(y_perm, ys, inv, w, T, k, renorm=True)
    b = O.combine(y_perm, ys, inv, w * 7.5, T, k, renorm=True)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=0)
    for t in range(T):
        tot = sum(w[t, j] for j in range(k))
        for h in range(H):
            ref = ys[t, h] + sum(w[t, j] / tot * y_perm[inv[t * k + j], h] for j in range(k))
            assert abs(a[t, h] - ref) < 1e-14
    # without renorm the same weights are used as they are
    assert not np.allclose(O.combine(y_perm, ys, inv, w, T, k), a)


def test_combine_bruteforce():
    g = np.random.default_rng(9)
    T, k, H = 4, 2, 5
    y_perm = g.standard_normal((T * k, H))
    ys = g.standard_normal((T, H))
    inv = g.permutation(T * k).astype(np.int32)
    w = g.uniform(size=(T, k))
    out = O.combine(y_perm, ys, inv, w, T, k)
    for t in range(T):
        for h in range(H):
            ref = ys[t, h] + sum(w[t, j] * y_perm[inv[t * k + j], h] for j in range(k))
            assert abs(out[t, h] - ref) < 1e-14


def test_rmsnorm_identity():
    g = np.random.default_rng(10)
    y = g.standard_normal((5, 64)) * np.array([[1e-4], [1e-2], [1], [10], [0.0]])
    eps = 1e-6
    r = O.rmsnorm(y, eps)
    ms = np.mean(y * y, axis=1)
    np.testing.assert_allclose(np.mean(r * r, axis=1), ms / (ms + eps), rtol=1e-12, atol=0)
