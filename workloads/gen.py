"""numpy generators: every tensor of every workload from one root seed.

Each tensor is drawn from its own PCG64 stream, keyed by
(config id, tensor kind, layer, expert, matrix, batch) through
numpy's SeedSequence spawn keys, so any single expert matrix of any layer can
be regenerated alone (the 42-layer stack does not fit in host memory).
"""
from __future__ import annotations

import numpy as np

from .configs import MoEConfig

ROOT_SEED = 0

# tensor kinds (part of the spawn key)
T_X, T_ROUTER_W, T_ROUTER_B, T_EXPERT, T_SHARED, T_CODES, T_SCALES, T_PERM, \
    T_DEAD = range(9)

GATE, UP, DOWN = 0, 1, 2


def seed_seq(cfg: MoEConfig, kind: int, layer: int = 0, expert: int = 0,
             matrix: int = 0, batch: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence(
        ROOT_SEED, spawn_key=(cfg.cfg_id, kind, layer, expert, matrix, batch))


def rng(cfg: MoEConfig, kind: int, **key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq(cfg, kind, **key)))


def torch_seed(cfg: MoEConfig, kind: int, **key) -> int:
    """A 63-bit seed for torch generators, from the same spawn key."""
    return int(seed_seq(cfg, kind, **key).generate_state(1, np.uint64)[0]
               & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def normal16(g: np.random.Generator, shape, std: float) -> np.ndarray:
    """N(0, std^2) drawn in float32, then stored as fp16."""
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)
            ).astype(np.float16)


def matrix_shape(cfg: MoEConfig, matrix: int):
    """[out, in]: gate/up are [F, H]; down is [H, F]."""
    return (cfg.ffn, cfg.hidden) if matrix in (GATE, UP) else (cfg.hidden, cfg.ffn)


def activations(cfg: MoEConfig, batch: int = 0, layer: int = 0, tokens=None):
    T = cfg.tokens if tokens is None else tokens
    return normal16(rng(cfg, T_X, layer=layer, batch=batch), (T, cfg.hidden), cfg.x_std)


def router_bias(cfg: MoEConfig, layer: int = 0):
    """Per-expert fp32 bias: alpha * ln(Zipf pmf of the expert's seeded rank),
    plus dead experts at a large negative bias; None when unbiased."""
    if not cfg.has_bias:
        return None
    E = cfg.num_experts
    b = np.zeros(E, dtype=np.float64)
    if cfg.zipf_alpha:
        z = np.arange(1, E + 1, dtype=np.float64) ** (-cfg.zipf_s)
        z /= z.sum()
        pi = rng(cfg, T_PERM, layer=layer).permutation(E)
        b = cfg.zipf_alpha * np.log(z[pi])
    if cfg.dead_experts:
        dead = rng(cfg, T_DEAD, layer=layer).choice(E, cfg.dead_experts, replace=False)
        b[dead] = cfg.dead_bias
    return b.astype(np.float32)


def router(cfg: MoEConfig, layer: int = 0):
    std = cfg.router_std if cfg.router_std is not None else cfg.hidden ** -0.5
    w = normal16(rng(cfg, T_ROUTER_W, layer=layer), (cfg.num_experts, cfg.hidden), std)
    return w, router_bias(cfg, layer)


def expert_master(cfg: MoEConfig, layer: int, expert: int, matrix: int):
    """fp16 master weight of one expert matrix, N(0, weight_std^2)."""
    return normal16(rng(cfg, T_EXPERT, layer=layer, expert=expert, matrix=matrix),
                    matrix_shape(cfg, matrix), cfg.weight_std)


def shared_expert(cfg: MoEConfig, layer: int = 0):
    """fp16 shared expert (Wg [Fs,H], Wu [Fs,H], Wd [H,Fs]), or None."""
    if not cfg.shared_ffn:
        return None
    Fs, H = cfg.shared_ffn, cfg.hidden
    return tuple(normal16(rng(cfg, T_SHARED, layer=layer, matrix=m), shp, cfg.shared_std)
                 for m, shp in ((GATE, (Fs, H)), (UP, (Fs, H)), (DOWN, (H, Fs))))


# Code distribution of int4-quantized N(0, sigma) weights: with 128-weight
# groups and scale max|w|/7, the code of a weight is about w * 7 / max|w|; the
# largest of 128 |N(0,1)| draws is 2.7 on average (2.2 .. 3.5 in practice),
# so the codes are close to a normal with standard deviation 7 / 2.7 = 2.6,
# rounded and clipped, and the scales about sigma * 2.7 / 7 (sigma * 0.33 .. 0.48).
CODE_STD = 2.6
SCALE_LO, SCALE_HI = 0.33, 0.48


def expert_codes(cfg: MoEConfig, layer: int, expert: int, matrix: int):
    """Packed int4 bytes and fp16 scales drawn directly (no quantizer), with
    the distribution that quantizing N(0, weight_std) masters produces.

    Each nibble is an independent draw u = clip(rint(CODE_STD * z), -7, 7) + 8
    with z ~ N(0, 1); a byte holds two such nibbles.  Because every nibble is
    drawn independently with the same law, the bytes have that law in any
    storage layout.  Scales are weight_std * U(SCALE_LO, SCALE_HI).  Used
    where drawing and quantizing fp16 masters on the host would take too long
    (full-size parity, the CPU baseline).
    """
    out_dim, in_dim = matrix_shape(cfg, matrix)
    g = rng(cfg, T_CODES, layer=layer, expert=expert, matrix=matrix)
    z = g.standard_normal((2, out_dim, in_dim // 2), dtype=np.float32)
    u = (np.clip(np.rint(z * np.float32(CODE_STD)), -7, 7) + 8).astype(np.uint8)
    packed = u[0] | (u[1] << 4)
    s = (cfg.weight_std * g.uniform(SCALE_LO, SCALE_HI,
                                    size=(out_dim, in_dim // cfg.group_size))).astype(np.float16)
    return packed, s
