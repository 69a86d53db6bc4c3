"""The no-allocation attention entry point against the workspace one (GPU).

csa_sparse_attn_decode_noalloc keeps its split partials in the library's
static device array instead of a caller workspace; it runs the same kernels,
so its output must equal csa_sparse_attn_decode's bit for bit.  Calls in a
row: the second on a smaller input (the array keeps the first call's
partials), a third on a shape that needs no partials, then the first shape
again.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_csa_amd import csa as C
from sparse_attention_decode_csa_amd import inputs as I
from tests import _util as U

pytestmark = pytest.mark.gpu


def _case(cid, **kw):
    cfg = I.CONFIGS[cid]
    sh = cfg.shape.replace(**kw)
    inp = I.make_inputs(cid, shape=sh)
    jobs = oracle.JOB_ATTN if cfg.supplied_topk else oracle.JOB_SCORE | oracle.JOB_TOPK | oracle.JOB_ATTN
    ref = oracle.run(sh, inp, jobs=jobs, nthreads=8)
    d = C.to_device(inp, sh)
    d["topk_idx"] = torch.from_numpy(ref["topk_idx"]).cuda()
    return sh, d, ref


def _both(sh, d):
    scale = I.softmax_scale(sh)
    bufs = C.alloc_outputs(sh)
    args = (d["q"], d["k_win"], d["v_win"], d["k_cmp"], d["v_cmp"], d["topk_idx"], d["start_pos"],
            d["rope_cos"], d["rope_sin"], scale)
    C.sparse_attn_decode(sh, *args, bufs["out"], bufs["attn_ws"])
    out_na = torch.full_like(bufs["out"], float("nan"))
    C.sparse_attn_decode_noalloc(sh, *args, out_na)
    torch.cuda.synchronize()
    return bufs["out"].float().cpu().numpy(), out_na.float().cpu().numpy()


def test_noalloc_equals_workspace_entry_point():
    assert torch.cuda.is_available()
    big = _case(4)              # 128 tokens, 5 splits each
    small = _case(4, batch=8)   # 16 tokens, 5 splits each
    token = _case(2)            # one workgroup per token: no partials at all
    assert C.sparse_attn_workspace_bytes(big[0]) > C.sparse_attn_workspace_bytes(small[0]) > 0
    assert C.sparse_attn_workspace_bytes(token[0]) == 0
    for sh, d, ref in (big, small, token, big):
        want, got = _both(sh, d)
        assert np.array_equal(got, want), "no-alloc output differs from the workspace entry point"
        U.compare_outputs(sh, got, ref["out"])
