"""bench.py's host side on the CPU: the one-GPU refusal and the algorithmic
work counts its roofline divides by, on hand-worked tiny shapes."""
import json
import os
import subprocess
import sys

import numpy as np

from sparse_attention_decode_csa_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def tiny(**kw):
    base = dict(batch=1, q_per_req=2, ratio=4, n_cap=64, topk=4, win=3, w_cap=4, heads=2,
                head_dim=4, rope_dim=0, idx_heads=2, idx_dim=8, out_groups=1, max_len=256,
                dtype=I.BF16)
    base.update(kw)
    return I.Shape(**base)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 1" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_score_bytes_hand_worked():
    sh = tiny()
    # positions 40 and 41: 10 visible rows each, both past K = 4
    #   keys 10 rows x 16 B (read once per request) + scores 2 x 10 x 4 B
    #   + queries 2 tokens x 2 heads x (16 B + a 4-byte weight)
    assert bench.score_bytes(sh, np.array([40])) == 160 + 80 + 80
    # FP8 keys: a row is 8 codes plus its 4-byte scale
    assert bench.score_bytes(sh, np.array([40]), "fp8") == 10 * 12 + 80 + 80
    # positions 15 and 16: 4 visible rows, both within K: nothing is scored
    assert bench.score_bytes(sh, np.array([15])) == 0
    # positions 19 and 20: 5 rows each; the keys of the longer row count once
    assert bench.score_bytes(sh, np.array([19])) == 5 * 16 + 2 * 5 * 4 + 80
    assert bench.score_flops(sh, np.array([40])) == 2 * (2 * 8 * 2 * 10)


def test_topk_bytes_hand_worked():
    sh = tiny()
    # each token writes K indices; a scored token also reads its row of scores
    assert bench.topk_bytes(sh, np.array([40])) == 2 * (4 * 4 + 10 * 4)
    assert bench.topk_bytes(sh, np.array([15])) == 2 * 4 * 4


def test_attn_bytes_counts_distinct_rows_per_request():
    sh = tiny(n_cap=8, topk=3)
    # token 0 at p = 5: window positions 3..5 -> ring slots 3, 0, 1
    # token 1 at p = 6: window positions 4..6 -> ring slots 0, 1, 2   (union: 4 rows)
    # lists {1, 2} and {2, 7} (99 lies past n_cap: padding)            (union: 3 rows)
    lists = np.array([[[1, 2, -1], [2, 7, 99]]], dtype=np.int32)
    total, attended = bench.attn_bytes(sh, np.array([5]), lists)
    row = 2 * 4 * 2                       # K and V rows of 4 bf16
    qo = 2 * 2 * 4 * 2 * 2                # q in and out, 2 tokens x 2 heads
    assert total == (4 + 3) * row + qo + 2 * 3 * 4
    assert attended == (3 + 2) + (3 + 2)
