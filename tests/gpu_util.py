"""Helpers shared by the GPU parity tests.

Inputs come from the seeded generators in workloads/ and, where the method's
own offline step is needed (fp16 masters -> int4 codes), from the oracle's
quantizer; expected values come from the oracle only.  The HIP path is
reached through the C ABI (w4_group_quantized_amd binding).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from workloads import gen as G

gpu = pytest.mark.gpu


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(dev())


def tol_check(gpu_vals, ref, what="", rel=1e-2, abs_=1e-3):
    """max|gpu - oracle| <= rel * max|oracle| + abs."""
    g = np.asarray(gpu_vals, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    err = np.abs(g - r).max() if r.size else 0.0
    bound = rel * (np.abs(r).max() if r.size else 0.0) + abs_
    assert err <= bound, f"{what}: max err {err:.3e} > bound {bound:.3e}"
    return err, bound


def quantized_experts(cfg, layer=0, experts=None):
    """Oracle-quantized expert weights from fp16 masters, stacked per matrix.

    Returns dict of numpy arrays gate_q [E,F,H/2], gate_s [E,F,H/gs], ...
    and the per-expert tuple list the oracle takes."""
    E = cfg.num_experts
    ids = range(E) if experts is None else experts
    mats = {n: [] for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}
    per_expert = []
    for e in ids:
        tup = []
        for m, name in ((G.GATE, "gate"), (G.UP, "up"), (G.DOWN, "down")):
            q, s = O.group_quantize(G.expert_master(cfg, layer, e, m), cfg.group_size)
            p, ss = O.pack_w4(q), O.pack_scales(s)
            mats[name + "_q"].append(p)
            mats[name + "_s"].append(ss)
            tup += [p, ss]
        per_expert.append(tuple(tup))
    return {k: np.stack(v) for k, v in mats.items()}, per_expert


def coded_experts(cfg, layer=0):
    """Directly drawn packed codes + scales (no quantizer), stacked per matrix."""
    mats = {n: [] for n in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")}
    per_expert = []
    for e in range(cfg.num_experts):
        tup = []
        for m, name in ((G.GATE, "gate"), (G.UP, "up"), (G.DOWN, "down")):
            p, s = G.expert_codes(cfg, layer, e, m)
            mats[name + "_q"].append(p)
            mats[name + "_s"].append(s)
            tup += [p, s]
        per_expert.append(tuple(tup))
    return {k: np.stack(v) for k, v in mats.items()}, per_expert


def shared_w8(shared):
    """The fp16 shared expert quantized to 8 bits by the oracle: the stored
    ((q, s), (q, s), (q, s)) numpy arrays for the device, and the float64
    dequantized (Wg, Wu, Wd) the oracle's SwiGLU takes."""
    stored, deq = [], []
    for w in shared:
        q, s = O.group_quantize(w, 128, bits=8)
        p, ss = O.pack_w8(q), O.pack_scales(s)
        stored.append((p, ss))
        deq.append(O.dequant_w8(p, ss))
    return tuple(stored), tuple(deq)


def make_gpu_layer(cfg, mats, wr, b, shared, w8=None):
    """w8: the stored arrays of an 8-bit shared expert (shared is then None)."""
    from w4_group_quantized_amd import W4MoELayer
    d = {k: to_dev(v) for k, v in mats.items()}
    sh = tuple(to_dev(w) for w in shared) if shared is not None else None
    s8 = tuple((to_dev(q), to_dev(s)) for q, s in w8) if w8 is not None else None
    layer = W4MoELayer(cfg.top_k, to_dev(wr), to_dev(b) if b is not None else None,
                       d["gate_q"], d["gate_s"], d["up_q"], d["up_s"], d["down_q"], d["down_s"],
                       shared=sh, shared_w8=s8)
    return layer


def route_compare(idx_gpu, logits_ref, k, gap=1e-6):
    """Top-k indices must equal the oracle's ordered lists exactly, except at
    positions where the GPU's expert and the oracle's differ by at most `gap`
    in float64 logit (a reported tie, oracle.tie_excused).  Returns the
    boolean mask of tokens that differ (all of them excused)."""
    idx_gpu = np.asarray(idx_gpu)
    differs, excused = O.tie_excused(idx_gpu, logits_ref, gap)
    bad = differs & ~excused
    assert not bad.any(), f"top-k mismatch on tokens {np.nonzero(bad)[0][:10]} (not a tie <= {gap})"
    if differs.any():
        print(f"[reported] {int(differs.sum())} token(s) differ at a tie <= {gap}")
    return differs


def on_gpu_selection(ref, idx_gpu, rerun, k):
    """Check the GPU's top-k against the oracle run `ref` (route_compare), and
    return the oracle layer to compare outputs with: `ref` itself when the
    selections agree, else rerun(idx_gpu), the oracle evaluated on the GPU's
    own selection, so that every token's output is compared."""
    differs = route_compare(idx_gpu, ref["logits"], k)
    return rerun(np.asarray(idx_gpu)) if differs.any() else ref
