"""The decode step captured in a HIP graph and replayed (GPU).

Every call of the step is a kernel launch on the caller's stream with no
allocation, copy or memset, so the whole step can be captured once
(torch.cuda.CUDAGraph over the C-ABI calls) and replayed.  Each replay runs
on new queries, copied into the captured input buffers between replays, with
eager steps of the library in between; every replay must equal the eager step
on the same inputs bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

from sparse_attention_decode_csa_amd import csa as C
from sparse_attention_decode_csa_amd import inputs as I

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _outputs(bufs):
    return {k: bufs[k].clone() for k in ("scores", "topk_idx", "out")}


def _same(a, b):
    for k in ("scores", "topk_idx", "out"):
        x, y = a[k].cpu(), b[k].cpu()
        if k == "scores":
            assert torch.equal(torch.isnan(x), torch.isnan(y)), k
            x, y = torch.nan_to_num(x), torch.nan_to_num(y)
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y), k


@pytest.mark.parametrize("cid", [3, 2, 4])
def test_graph_replay_equals_eager(cid):
    # config 3: scoring, Top-K and the split attention kernels; config 2: the
    # one-workgroup-per-token attention on supplied lists; config 4: the wide
    # Top-K step the benchmark times
    cfg = I.CONFIGS[cid]
    sh = cfg.shape
    dev = C.to_device(I.make_inputs(cid), sh)
    bufs = C.alloc_outputs(sh)
    scale = I.softmax_scale(sh)
    names = ("q", "q_idx", "w")
    qsets = [{n: torch.roll(dev[n], shifts=r + 1, dims=0).contiguous() for n in names}
             for r in range(REPLAYS)]
    C.step(sh, dev, bufs, scale, supplied_topk=cfg.supplied_topk)   # eager first call
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        C.step(sh, dev, bufs, scale, stream=torch.cuda.current_stream(),
               supplied_topk=cfg.supplied_topk)
    torch.cuda.synchronize()
    outs = []
    for r in range(REPLAYS):
        for n in names:
            dev[n].copy_(qsets[r][n])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(bufs)
        eager = C.alloc_outputs(sh)
        C.step(sh, dev, eager, scale, supplied_topk=cfg.supplied_topk)
        torch.cuda.synchronize()
        _same(got, eager)
        outs.append(got["out"].cpu())
    # the replays really ran on their new queries
    assert not torch.equal(outs[0], outs[-1])


def test_graph_replay_no_alloc_attention():
    # the entry point for callers that cannot allocate, captured: its split
    # partials live in the library's static array
    cid = 3
    cfg = I.CONFIGS[cid]
    sh = cfg.shape
    dev = C.to_device(I.make_inputs(cid), sh)
    bufs = C.alloc_outputs(sh)
    scale = I.softmax_scale(sh)
    C.step(sh, dev, bufs, scale)   # lists for the attention
    torch.cuda.synchronize()
    assert C.sparse_attn_workspace_bytes(sh) > 0
    args = (dev["q"], dev["k_win"], dev["v_win"], dev["k_cmp"], dev["v_cmp"], bufs["topk_idx"],
            dev["start_pos"], dev["rope_cos"], dev["rope_sin"], scale)
    out = torch.full_like(bufs["out"], float("nan"))
    C.sparse_attn_decode_noalloc(sh, *args, out)   # first call: looks up the array
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        C.sparse_attn_decode_noalloc(sh, *args, out, stream=torch.cuda.current_stream())
    for r in range(REPLAYS):
        dev["q"].copy_(torch.roll(dev["q"], shifts=1, dims=0))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = torch.empty_like(out)
        C.sparse_attn_decode(sh, *args, want, bufs["attn_ws"])
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16).cpu(), want.view(torch.int16).cpu()), f"replay {r}"
