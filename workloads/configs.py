"""The MoE-layer workloads, with the input recipe of each.

Shapes and distributions follow the workload descriptions of this project;
the expert shape of the fine-grained layers (288 routed experts + 1 shared,
top-8, 42 MoE layers) is the GLM-5.3-Flash shape of [P5] §01, the coarse
experts (~2.4B parameters, top-4) follow the capacity account of [P1] §1.2,
and the 20%-of-experts-take-80%-of-selections skew follows [P1] §2.1.

Readings (the descriptions leave these open):
  * router bias "Zipf": b[e] = alpha * ln z[pi(e)], z = Zipf(1.1) pmf over
    ranks 1..E, pi a seeded permutation; alpha = 0.7 for the fine-grained
    decode layers (logit std ~1.28 from N(0,0.02) router weights) and 0.2 for
    the prefill layer (logit std ~1), where 4 seeded experts additionally get
    b = -8 so that near-empty segments occur.
  * "uniform-random routing logits" (coarse layer): router weights
    N(0, 1/H) and no bias, so every expert is equally likely.
  * expert weights N(0, 0.02) where not stated; shared expert fp16 N(0, 0.02).
  * the 512-expert decode layer (the second model of [P5] §09: 48 layers, 512
    routed experts, 10 routed + 1 shared per token, expert intermediate size
    640) gets hidden 2560: the page gives no width, and 125B parameters over
    48 layers x 512 experts x 3 matrices x 640 leave at most ~2650 for the
    experts alone, so the nearest common model width below it; the shared
    expert has the routed experts' shape (ffn 640); 8 decode tokens as in the
    288-expert layer; the same Zipf(1.1) bias recipe, with alpha = 0.5 so
    that again about 20% of the experts take about 80% of the selections
    (logit std ~1.01 from N(0,0.02) router weights at H = 2560).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int
    num_experts: int
    hidden: int
    ffn: int
    top_k: int
    tokens: int
    shared_ffn: int = 0          # 0 = no shared expert
    layers: int = 1
    router_std: float = 0.02     # None -> 1/sqrt(hidden)
    zipf_alpha: float = 0.0      # 0 = no bias
    zipf_s: float = 1.1
    dead_experts: int = 0        # experts whose bias is set to dead_bias
    dead_bias: float = -8.0
    weight_std: float = 0.02
    shared_std: float = 0.02
    x_std: float = 1.0
    rms_eps: float = 1e-6        # used between stacked layers only
    group_size: int = 128        # int4 quantization group along in_features (64 / 128 / 256)
    shared_bits: int = 16        # shared expert weights: fp16, or 8-bit g128

    @property
    def has_bias(self) -> bool:
        return self.zipf_alpha != 0.0 or self.dead_experts > 0

    def expert_packed_bytes(self) -> int:
        return 3 * self.hidden * self.ffn // 2

    def expert_scale_bytes(self) -> int:
        return 3 * self.hidden * self.ffn // self.group_size * 2

    def expert_bytes(self) -> int:
        return self.expert_packed_bytes() + self.expert_scale_bytes()

    def shared_bytes(self) -> int:
        n = 3 * self.hidden * self.shared_ffn
        return n * 2 if self.shared_bits == 16 else n + n // 128 * 2


CONFIGS = {
    "tiny": MoEConfig("tiny", 1, num_experts=8, hidden=256, ffn=512, top_k=2,
                      tokens=16),
    "decode_fine": MoEConfig("decode_fine", 2, num_experts=288, hidden=4096,
                             ffn=1536, top_k=8, tokens=8, shared_ffn=1536,
                             zipf_alpha=0.7),
    "decode_coarse": MoEConfig("decode_coarse", 3, num_experts=16, hidden=12288,
                               ffn=65536, top_k=4, tokens=16, router_std=None,
                               weight_std=0.01),
    "prefill": MoEConfig("prefill", 4, num_experts=128, hidden=4096, ffn=2048,
                         top_k=8, tokens=8192, router_std=None, zipf_alpha=0.2,
                         dead_experts=4),
    "decode_stack": MoEConfig("decode_stack", 5, num_experts=288, hidden=4096,
                              ffn=1536, top_k=8, tokens=16, shared_ffn=1536,
                              layers=42, zipf_alpha=0.7),
    "decode_fine512": MoEConfig("decode_fine512", 6, num_experts=512, hidden=2560,
                                ffn=640, top_k=10, tokens=8, shared_ffn=640,
                                zipf_alpha=0.5),
}


def get_config(name: str, **overrides) -> MoEConfig:
    base = CONFIGS[name]
    if not overrides:
        return base
    d = dict(base.__dict__)
    d.update(overrides)
    return MoEConfig(**d)
