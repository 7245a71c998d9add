"""Pins of the C float64 reference products (oracle/w4_matvec.c) used for
full-size checks: exhaustive fp16 decoding, exact integer arithmetic, and
agreement with the numpy oracle's dequantize-then-multiply."""
import numpy as np
import pytest

import oracle as O
from oracle import cref as C


def test_fp16_decoding_exhaustive():
    """Code +1 (nibble 9) times every fp16 scale pattern returns the scale:
    the C decoder must agree with IEEE binary16 for all 65536 patterns."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    s_log = bits.view(np.float16).reshape(-1, 1).repeat(2, axis=1)   # [65536, 2] groups
    rows = s_log.shape[0]
    q = O.pack_w4(np.ones((rows, 256), dtype=np.int8))
    st = O.pack_scales(s_log)
    got = np.concatenate([C.dequant_rows(q, st, r, r + 4096)[:, 0]
                          for r in range(0, rows, 4096)])
    want = s_log[:, 0].astype(np.float64)
    finite = np.isfinite(want)
    np.testing.assert_array_equal(got[finite], want[finite])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    np.testing.assert_array_equal(got[np.isinf(want)], want[np.isinf(want)])


def test_dequant_rows_equals_numpy_oracle():
    g = np.random.default_rng(21)
    q = g.integers(0, 256, size=(48, 384), dtype=np.uint8)          # every code
    s = g.uniform(1e-4, 1e-1, size=(48, 6)).astype(np.float16)
    s[3, 2] = 0
    np.testing.assert_array_equal(C.dequant_rows(q, s, 0, 48), O.dequant(q, s))
    np.testing.assert_array_equal(C.dequant_rows(q, s, 16, 32), O.dequant(q, s)[16:32])


def test_matvec_exact_on_integer_inputs():
    """Power-of-two scales and small-integer activations: every product and
    partial sum is exact in float64, so both implementations agree exactly
    with an integer matmul."""
    g = np.random.default_rng(22)
    qi = g.integers(-8, 8, size=(32, 512)).astype(np.int8)
    sl = (2.0 ** g.integers(-6, 0, size=(32, 4))).astype(np.float16)
    x = g.integers(-3, 4, size=(5, 512)).astype(np.float64)
    ref = (x.astype(np.int64) @ qi.astype(np.int64).T).astype(np.float64)   # no scales yet
    W = qi.astype(np.float64) * np.repeat(sl.astype(np.float64), 128, axis=1)
    exact = x @ W.T
    got = C.w4_matvec(O.pack_w4(qi), O.pack_scales(sl), x)
    np.testing.assert_array_equal(got, exact)
    # with unit scales the result is the integer matmul itself
    ones = np.ones_like(sl)
    np.testing.assert_array_equal(C.w4_matvec(O.pack_w4(qi), O.pack_scales(ones), x), ref)


@pytest.mark.parametrize("out_dim,in_dim,ntok", [(16, 128, 1), (64, 1024, 7), (48, 384, 3)])
def test_matvec_matches_numpy_oracle(out_dim, in_dim, ntok):
    g = np.random.default_rng(out_dim + in_dim)
    q = g.integers(0, 256, size=(out_dim, in_dim // 2), dtype=np.uint8)
    s = g.uniform(1e-3, 3e-2, size=(out_dim, in_dim // 128)).astype(np.float16)
    x = g.standard_normal((ntok, in_dim))
    ref = x @ O.dequant(q, s).T
    np.testing.assert_allclose(C.w4_matvec(q, s, x), ref, rtol=1e-12, atol=1e-13)


def test_expert_ffn_matches_numpy_oracle():
    g = np.random.default_rng(23)
    H, F = 256, 384
    mats = []
    for out_dim, in_dim in ((F, H), (F, H), (H, F)):
        mats += [g.integers(0, 256, size=(out_dim, in_dim // 2), dtype=np.uint8),
                 g.uniform(1e-3, 2e-2, size=(out_dim, in_dim // 128)).astype(np.float16)]
    X = g.standard_normal((4, H))
    np.testing.assert_allclose(C.expert_ffn_w4_c(X, *mats), O.expert_ffn_w4(X, *mats),
                               rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("gs", [64, 256])
def test_matvec_and_dequant_other_group_sizes(gs):
    """Groups of 64 and 256 columns: the C decoder reads the group size off
    the scale shape and agrees with the numpy oracle (exactly for the
    dequantized weights), and with exact arithmetic on integer inputs."""
    g = np.random.default_rng(gs)
    out_dim, in_dim = 32, 512
    q = g.integers(0, 256, size=(out_dim, in_dim // 2), dtype=np.uint8)
    s = g.uniform(1e-3, 3e-2, size=(out_dim, in_dim // gs)).astype(np.float16)
    np.testing.assert_array_equal(C.dequant_rows(q, s, 0, out_dim), O.dequant(q, s, gs))
    x = g.standard_normal((3, in_dim))
    np.testing.assert_allclose(C.w4_matvec(q, s, x), x @ O.dequant(q, s, gs).T,
                               rtol=1e-12, atol=1e-13)
    qi = g.integers(-8, 8, size=(out_dim, in_dim)).astype(np.int8)
    sl = (2.0 ** g.integers(-6, 0, size=(out_dim, in_dim // gs))).astype(np.float16)
    xi = g.integers(-3, 4, size=(4, in_dim)).astype(np.float64)
    W = qi.astype(np.float64) * np.repeat(sl.astype(np.float64), gs, axis=1)
    np.testing.assert_array_equal(C.w4_matvec(O.pack_w4(qi), O.pack_scales(sl), xi), xi @ W.T)


def test_unsupported_shapes_are_refused():
    q = np.zeros((16, 64), np.uint8)
    with pytest.raises(ValueError):
        C.w4_matvec(q, np.zeros((16, 3), np.float16), np.zeros((1, 128)))   # 128/3 columns
    with pytest.raises(ValueError):
        C.w4_matvec(q, np.zeros((16, 4), np.float16), np.zeros((1, 128)))   # groups of 32
