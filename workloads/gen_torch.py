"""Device-side draws for full-size workloads (torch's seeded generators).

Only random draws: packed int4 codes and fp16 scales drawn directly, with the
distribution of workloads.gen.expert_codes, one stream per (config, layer,
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
    codes uint8 [E, out, in/2] (every byte value equally likely) and scales fp16
    [E, out, in/group_size] = weight_std * U(0.15, 0.30)."""
    out = {}
    for m, name in ((G.GATE, "gate"), (G.UP, "up"), (G.DOWN, "down")):
        out_dim, in_dim = G.matrix_shape(cfg, m)
        g = torch.Generator(device=device)
        g.manual_seed(G.torch_seed(cfg, G.T_CODES, layer=layer, matrix=m, batch=weight_set))
        E = cfg.num_experts
        q = torch.empty((E, out_dim, in_dim // 2), dtype=torch.uint8, device=device)
        for e in range(E):     # one expert at a time keeps int64 temporaries small
            q[e] = torch.randint(0, 256, (out_dim, in_dim // 2), generator=g, device=device,
                                 dtype=torch.uint8)
        s = (cfg.weight_std * (0.15 + 0.15 * torch.rand((E, out_dim, in_dim // cfg.group_size),
                                                          generator=g,
                                                          device=device))).to(torch.float16)
        out[name + "_q"], out[name + "_s"] = q, s
    return out
