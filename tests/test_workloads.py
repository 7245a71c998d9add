"""The input recipes: the routing skew the workload descriptions ask for
(about 20% of the experts taking about 80% of the selections on the
fine-grained layers, segment sizes from ~0 to ~2000 rows on the prefill
layer), measured with the oracle's router on the generated inputs."""
import numpy as np
import pytest

import oracle as O
from workloads import get_config
from workloads import gen as G


@pytest.mark.parametrize("name,batches", [("decode_fine", 40), ("decode_fine512", 40)])
def test_fine_grained_layers_route_80_percent_to_20_percent_of_experts(name, batches):
    cfg = get_config(name)
    wr, b = G.router(cfg)
    cnt = np.zeros(cfg.num_experts)
    for bt in range(batches):
        idx, _, _ = O.route(G.activations(cfg, batch=bt), wr, b, cfg.top_k)
        cnt += np.bincount(idx.ravel(), minlength=cfg.num_experts)
    top = np.sort(cnt)[::-1][: cfg.num_experts // 5].sum() / cnt.sum()
    assert 0.75 <= top <= 0.85, top


def test_prefill_segment_sizes_span_near_empty_to_about_two_thousand():
    cfg = get_config("prefill")
    wr, b = G.router(cfg)
    idx, _, _ = O.route(G.activations(cfg, batch=0), wr, b, cfg.top_k)
    seg = np.bincount(idx.ravel(), minlength=cfg.num_experts)
    assert seg.min() <= 16 and 1500 <= seg.max() <= 2600, (seg.min(), seg.max())
