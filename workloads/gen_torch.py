"""Device-side draws for full-size workloads (torch's seeded generators).

Only random draws: packed int4 codes and fp16 scales drawn directly, with the
law of workloads.gen.expert_codes (that of quantized N(0, sigma) weights), one stream per (config, layer,
matrix) keyed like the numpy generators.  Used where the weights are too
large to draw on the host (the 42-layer stack holds 119 GB); the oracle side
reads back the experts it needs.
"""
from __future__ import annotations

import torch

from .configs import MoEConfig
from . import gen as G


def layer_codes(cfg: MoEConfig, layer: int, device, weight_set: int = 0):
    """dict gate_q/gate_s/up_q/up_s/down_q/down_s for all experts of a layer:
    codes uint8 [E, out, in/2] and scales fp16 [E, out, in/group_size] with
    the law of workloads.gen.expert_codes (each nibble an independent
    clipped, rounded normal draw of standard deviation gen.CODE_STD; scales
    weight_std * U(gen.SCALE_LO, gen.SCALE_HI))."""
    out = {}
    for m, name in ((G.GATE, "gate"), (G.UP, "up"), (G.DOWN, "down")):
        out_dim, in_dim = G.matrix_shape(cfg, m)
        g = torch.Generator(device=device)
        g.manual_seed(G.torch_seed(cfg, G.T_CODES, layer=layer, matrix=m, batch=weight_set))
        E = cfg.num_experts
        q = torch.empty((E, out_dim, in_dim // 2), dtype=torch.uint8, device=device)
        for e in range(E):     # one expert at a time keeps the fp32 temporaries small
            z = torch.randn((2, out_dim, in_dim // 2), generator=g, device=device)
            u = (z.mul_(G.CODE_STD).round_().clamp_(-7, 7) + 8).to(torch.uint8)
            q[e] = u[0] | (u[1] << 4)
            del z, u
        lo, hi = G.SCALE_LO, G.SCALE_HI
        s = (cfg.weight_std * (lo + (hi - lo) * torch.rand(
            (E, out_dim, in_dim // cfg.group_size), generator=g, device=device))).to(torch.float16)
        out[name + "_q"], out[name + "_s"] = q, s
    return out
