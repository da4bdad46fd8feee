"""The seeded synthetic workloads have the routing structure of the layers
they stand in for (CPU, oracle routing on the generated logits):

- Mixtral-shaped (8 experts, top-2, learned-like gate): near-balanced, every
  expert within 10% of the mean load;
- Qwen3-shaped (128 experts, top-8, Zipf-skewed router bias): heavily
  skewed, with experts that receive no tokens at all (the empty-segment
  case every grouped kernel must handle) and a hot expert far above the
  mean.
"""
import numpy as np
import pytest

from oracle import moe_oracle as O
from synthetic import CONFIGS, generate_config


def _loads(name):
    c = CONFIGS[name]
    d = generate_config(c, seed=0, want=("logits",))
    assert d["logits"].shape == (c.T, c.E)
    assert d["logits"].dtype == np.float32
    idx, w = O.route_topk(d["logits"], c.k)
    cnt = np.bincount(idx.ravel(), minlength=c.E)
    assert cnt.sum() == c.T * c.k
    return c, cnt


def test_mixtral_routing_near_balanced():
    c, cnt = _loads("mixtral")
    mean = c.T * c.k / c.E
    assert cnt.min() >= 0.9 * mean and cnt.max() <= 1.1 * mean, cnt


@pytest.mark.parametrize("name", ["qwen3", "qwen3_long"])
def test_qwen3_routing_skewed_with_empty_experts(name):
    c, cnt = _loads(name)
    mean = c.T * c.k / c.E
    assert (cnt == 0).sum() >= 1, "no zero-token expert"
    assert cnt.max() >= 10 * mean, cnt.max()
