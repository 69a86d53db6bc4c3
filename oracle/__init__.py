"""CPU oracle of the CSA sparse-attention decode step (test infrastructure).

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product path never does: it runs the HIP
library or fails.
"""
from .csa_oracle import (JOB_ATTN, JOB_SCORE, JOB_TOPK, build, e4m3_value, n_vis, round_bf16,  # noqa: F401
                         run, run_paged, select_row, swa_writeback, unpage)
