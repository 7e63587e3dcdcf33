"""CPU checks of the seeded workload recipes against the rules they were chosen by."""
import dataclasses

import numpy as np

import workloads as W
from oracle import moe_oracle as orc


def _skew_counts(beta_list):
    """Expert loads of the skewed preset's seeded routing for each Zipf strength beta.
    The bias enters the logits last, so the bias-free fixed-order logits are computed
    once and each beta's bias is added in float32, as the router adds it."""
    cfg = W.preset("skew32_zipf_bf16")
    base = W.router_inputs(cfg, seed=0)
    logits0 = orc.router_logits(base["x"], base["wg"], cfg.dtype, None)
    out = {}
    for beta in beta_list:
        bias = W.router_inputs(dataclasses.replace(cfg, T=1, zipf_beta=beta), seed=0)["bias"]
        idx = orc.select_topk(logits0 + bias[None, :], cfg.k)
        out[beta] = np.bincount(idx.reshape(-1), minlength=cfg.E)
    return out


def test_skew_beta_is_the_smallest_meeting_the_rule():
    # rule: the hottest expert takes >= 24% of the assignments (top-4 caps it at 25%) and
    # at least one expert gets none; SKEW_BETA must be the smallest such beta of the grid
    grid = [1.5, 2.0, 2.5, 3.0]
    counts = _skew_counts(grid[:grid.index(W.SKEW_BETA) + 1])

    def meets(c):
        return c.max() / c.sum() >= 0.24 and (c == 0).sum() >= 1

    assert W.preset("skew32_zipf_bf16").zipf_beta == W.SKEW_BETA
    assert meets(counts[W.SKEW_BETA]), counts[W.SKEW_BETA]
    for beta in grid[:grid.index(W.SKEW_BETA)]:
        assert not meets(counts[beta]), (beta, counts[beta])


def test_router_inputs_match_generate():
    cfg = W.shrink(W.preset("skew32_zipf_bf16"), T=300, D=256, F=128)
    full = W.generate(cfg, seed=4)
    part = W.router_inputs(cfg, seed=4)
    for name in ("x", "wg", "bias"):
        np.testing.assert_array_equal(part[name], full[name])
