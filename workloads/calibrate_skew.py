"""Pick the strength of the Zipf router bias of the skewed preset.

Runs the oracle's routing on the seeded skewed inputs for beta in {1.5, 2, 2.5, 3}
and reports the largest expert's share of the assignments and the number of experts
left empty. The preset uses the smallest beta whose share is at least 24% (top-4
caps any expert at 25%) and that leaves at least one expert with no rows.

    python -m workloads.calibrate_skew
"""
import dataclasses

import numpy as np

import workloads
from oracle import moe_oracle


def main():
    base = workloads.preset("skew32_zipf_bf16")
    chosen = None
    for beta in (1.5, 2.0, 2.5, 3.0):
        cfg = dataclasses.replace(base, zipf_beta=beta)
        inp = workloads.generate(cfg)
        idx, _, _ = moe_oracle.route(inp["x"], inp["wg"], cfg.k, cfg.dtype, inp["bias"])
        counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
        share = counts.max() / counts.sum()
        empty = int((counts == 0).sum())
        print(f"beta={beta}: max share {share:.4f}, empty experts {empty}, counts {counts.tolist()}")
        if chosen is None and share >= 0.24 and empty >= 1:
            chosen = beta
    print("chosen beta:", chosen)


if __name__ == "__main__":
    main()
