"""Score rows past 32-bit offsets (GPU).

The decode-shaped score kernel writes a workgroup's score rows through 32-bit
buffer offsets while they stay below 2^31 bytes, and with 64-bit streaming
stores past that.  Here one workgroup holds 64 query tokens of one indexer
head over a cache of 2^23 + 4096 compressed rows: 2.1 GB of score rows.  The
first and the last token are checked against the oracle over every visible
row, and the rows past each token's visible count must stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_csa_amd import csa as C
from sparse_attention_decode_csa_amd import inputs as I
from tests import _util as U

pytestmark = pytest.mark.gpu


def test_score_rows_past_32bit_offsets():
    assert torch.cuda.is_available()
    S, n_cap = 64, (1 << 23) + 4096
    max_len = 4 * n_cap
    cfg = I.CONFIGS[3]
    sh = cfg.shape.replace(batch=1, q_per_req=S, idx_heads=1, idx_dim=64, n_cap=n_cap, topk=64,
                           max_len=max_len, w_cap=256)
    assert S * sh.idx_heads <= 64 and S * n_cap * 4 > 0x7FFFF000  # one workgroup, rows past 2^31 bytes
    sp = np.array([max_len - S], dtype=np.int32)
    inp = I.make_inputs(cfg, shape=sh, start_pos=sp, structure="none", indexer_only=True)
    d = {k: torch.from_numpy(inp[k].view(np.int16)).view(torch.bfloat16).cuda() for k in ("q_idx", "k_idx")}
    w = torch.from_numpy(inp["w"]).cuda()
    start = torch.from_numpy(sp).cuda()
    scores = torch.full((1, S, n_cap), float("nan"), dtype=torch.float32, device="cuda")
    C.indexer_score(sh, d["q_idx"], w, d["k_idx"], start, scores)
    torch.cuda.synchronize()
    print("case: 64 tokens x (2^23 + 4096) rows, tokens 0 and 63 against the oracle", flush=True)
    rows = [r for r in U.token_rows(sh, sp) if r[1] in (0, S - 1)]
    assert [r[1] for r in rows] == [0, S - 1] and rows[0][2] == n_cap - 16 and rows[1][2] == n_cap
    bound = U.score_error_bound(sh, inp, rows)
    for (b, s, n) in rows:
        got = scores[b, s].cpu().numpy()
        ref = oracle.run(sh, inp, jobs=oracle.JOB_SCORE, tokens=(s, s + 1), nthreads=8)["scores"][b, s]
        err = np.abs(got[:n].astype(np.float64) - ref[:n])
        assert np.all(err <= bound[(b, s)]), f"token {s}: score error above bound (worst {err.max():.3g})"
        assert np.isnan(got[n:]).all(), f"token {s}: rows past the visible count were written"
