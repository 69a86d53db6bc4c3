"""Which indexer key row the wide Top-K configuration's boundary tie copies.

    python tests/golden/config4_boundary_tie.py

The wide Top-K workload (64 requests, 2 query tokens each, 32768 compressed
rows, K = 1024, 1% duplicated key rows) also carries a tie that straddles the
selection boundary: the key row that its first query token ranks K-th is
copied to two rows below it and two above it.  Five rows then share the
boundary score; only the ranks above the boundary are left for them, so the
lower index decides which of the five are kept (the tie rule of the Top-K
item of "Fix: port the DeepSeek-V4 MoE, hc_pre and prefill fixes to DSpark",
description, and the reference-sort regression its review asks for).

That row is found here with the CPU oracle alone: it scores token (0, 0) on
the configuration's inputs drawn without the tie and selects; the rank-K row
is the member of the oracle's list with the lowest score, the highest index
among equal scores (the list is ordered by score, then by lower index).  The
printed row number is the one written into the configuration's structure in
the input generator; `tests/test_oracle_pins.py` re-derives it the same way.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from sparse_attention_decode_csa_amd import inputs as I  # noqa: E402

BASE_STRUCTURE = "dup:0.01"   # the wide Top-K configuration's structure before the tie


def rank_k_row(inp, shape, b=0, s=0):
    """The row that token (b, s) ranks K-th, from the oracle's scores and list."""
    t = b * shape.q_per_req + s
    ref = oracle.run(shape, inp, jobs=oracle.JOB_SCORE | oracle.JOB_TOPK, tokens=(t, t + 1),
                     nthreads=8)
    sel = ref["topk_idx"][b, s]
    sc = ref["scores"][b, s, sel].astype(np.float64)
    low = sel[sc == sc.min()]
    return int(low.max())


def main():
    cfg = I.CONFIGS[4]
    inp = I.make_inputs(cfg, structure=BASE_STRUCTURE)
    print(rank_k_row(inp, cfg.shape))


if __name__ == "__main__":
    main()
