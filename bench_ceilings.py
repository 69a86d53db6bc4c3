"""Memory-system ceilings beside the decode step's kernels, on one MI355X.

    python bench_ceilings.py [--config 4|3] [--reps 40] [--flush-mib 1024]

On the wide Top-K workload (config 4, the default: 64 requests x 2 query
tokens, 32768 compressed rows of 256 bytes per request, K = 1024, window 256)
or the long-context one (config 3: 16 requests x 1 token, 8192-16384 visible
rows, K = 512, window 128), this times, flushed
(1 GiB written and 512 MiB read before every launch, outside its events) and
hot (no flush; a GPU spin that touches no memory runs before each launch, so
that the host's launch overhead stays outside the events):

- the library's indexer score kernel, and probes that read the key pages it
  reads (the visible rows) and compute nothing: the score kernel's own LDS-DMA
  stream in address order and with the pages in a random order, and plain
  16-byte vector loads of as many bytes, one contiguous range per workgroup;
- the paged score kernel over a pool of 64-row blocks in a seeded random
  order, and the LDS-DMA stream reading the same pages through the same table;
- the library's Top-K kernel right after the score kernel (untimed) wrote its
  rows, and probes that only read those rows (whole rows): one 1024-thread
  workgroup per row (the Top-K's own load), one or 8 256-thread ones;
- the library's attention call, and a probe that gathers exactly its K and V
  rows (the step's own Top-K lists plus the window rows) 4 rows per wave and
  computes nothing, next to a sequential read of as many bytes.

The probes live in libcsa_ceilings.so (csrc/ceilings.hip); the decode path
never loads that library.  Prints one JSON line per measurement and a last
line with all of them.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CEILINGS_LIB = os.path.join(ROOT, "sparse_attention_decode_csa_amd", "libcsa_ceilings.so")
DMA_WG_BYTES = 131072
DMA_PAGE_BYTES = 16384
ROW_BYTES = 256
WORKLOADS = (4, 3)  # wide Top-K (the default), long context
SPIN_CYCLES = 400_000  # a GPU spin of about 0.2 ms before each hot launch
PAGE_ROWS = 64         # rows per block of the paged key pool (16 KiB of bf16 keys)


def load_ceilings() -> ctypes.CDLL:
    if not os.path.exists(CEILINGS_LIB):
        raise ImportError(f"{CEILINGS_LIB} is missing: build it with python -m sparse_attention_decode_csa_amd.build")
    L = ctypes.CDLL(CEILINGS_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.csa_ceiling_stream_dma.argtypes = [vp, i64, vp, i32, vp, vp]
    L.csa_ceiling_stream_vec.argtypes = [vp, i64, i32, i32, vp, vp]
    L.csa_ceiling_gather.argtypes = [vp, vp, i64, vp, i32, vp, vp]
    for f in (L.csa_ceiling_stream_dma, L.csa_ceiling_stream_vec, L.csa_ceiling_gather):
        f.restype = ctypes.c_int
    return L


def visible_key_pages(sh, start_pos, rows_per_page: int):
    """The key-cache pages (rows_per_page rows each, numbered b * pages_per_request
    + i) holding the rows the score kernel reads: per request, its first nmax
    rows, nmax the largest visible count among its tokens that do not fit
    Top-K.  Ascending, padded with copies of the last page to whole probe
    workgroups.  Also returns how many scores the step writes."""
    if sh.n_cap % rows_per_page:
        raise ValueError("n_cap must be a whole number of pages")
    bpr = sh.n_cap // rows_per_page
    vis, score_rows = [], 0
    for b in range(sh.batch):
        nmax = 0
        for s in range(sh.q_per_req):
            p = min(max(int(start_pos[b]) + s, 0), sh.max_len - 1)
            nv = min((p + 1) // sh.ratio, sh.n_cap)
            if nv > sh.topk:
                nmax = max(nmax, nv)
                score_rows += nv
        vis.extend(b * bpr + i for i in range(-(-nmax // rows_per_page)))
    if not vis:
        raise ValueError("no token of this step is scored")
    per_wg = DMA_WG_BYTES // DMA_PAGE_BYTES
    vis += [vis[-1]] * (-len(vis) % per_wg)
    return np.asarray(vis, dtype=np.int32), score_rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=40, help="timed launches per measurement and cache state")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--config", type=int, choices=WORKLOADS, default=WORKLOADS[0])
    args = ap.parse_args()

    import torch
    from sparse_attention_decode_csa_amd import csa as C
    from sparse_attention_decode_csa_amd import inputs as I

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    C.lib()
    P = load_ceilings()
    cfg = I.CONFIGS[args.config]
    sh = cfg.shape
    inp = I.make_inputs(args.config)
    dev = C.to_device(inp, sh)
    bufs = C.alloc_outputs(sh)
    scale = I.softmax_scale(sh)
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    print(f"# {cfg.name}: inputs uploaded", file=sys.stderr, flush=True)

    # the step's own Top-K lists (one step on the resident inputs)
    C.indexer_score(sh, dev["q_idx"], dev["w"], dev["k_idx"], dev["start_pos"], bufs["scores"], stream)
    C.topk(sh, bufs["scores"], dev["start_pos"], bufs["topk_idx"], bufs["topk_ws"], stream)
    torch.cuda.synchronize()

    scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device="cuda")
    clean = torch.ones((args.flush_mib << 20) // 8, dtype=torch.float32, device="cuda")

    def flush(k):
        scratch.fill_(k & 0x7F)
        clean.sum()

    results = []

    def timed(name, nbytes, launch, note="", pre=None):
        for mode in ("flushed", "hot"):
            ts = []
            for k in range(args.reps + 5):
                if mode == "flushed":
                    flush(k)
                else:
                    # keep the GPU busy (without touching memory) while the
                    # host queues the events and the launch, so the interval
                    # holds GPU time only
                    torch.cuda._sleep(SPIN_CYCLES)
                if pre is not None:
                    pre()  # untimed: what the step runs just before
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                launch()
                e1.record(stream)
                e1.synchronize()
                if k >= 5:
                    ts.append(e0.elapsed_time(e1) * 1e3)
            med, mn = float(np.median(ts)), float(np.min(ts))
            rec = {"measure": name, "cache": mode, "us_median": round(med, 2), "us_min": round(mn, 2),
                   "bytes": int(nbytes), "tb_s_median": round(nbytes / (med * 1e-6) / 1e12, 3),
                   "frac_of_8tbs": round(nbytes / (med * 1e-6) / 8e12, 3), "launches": args.reps}
            if note:
                rec["note"] = note
            results.append(rec)
            print(json.dumps(rec), flush=True)

    def ok(code, what):
        if code != 0:
            raise RuntimeError(f"{what} refused or failed ({code})")

    # ---- the key stream: the 16 KiB pages holding the rows the score kernel
    # reads (each request's visible rows, up to the most any of its tokens
    # that do not fit Top-K sees), padded to whole probe workgroups
    keys = dev["k_idx"]
    B = sh.batch
    rows_per_page = DMA_PAGE_BYTES // (sh.idx_dim * keys.element_size())
    bpr = sh.n_cap // rows_per_page
    vis, score_rows = visible_key_pages(sh, inp["start_pos"], rows_per_page)
    kbytes = vis.size * DMA_PAGE_BYTES
    d_vis = torch.from_numpy(vis).cuda()
    d_rand = torch.from_numpy(np.random.default_rng(5).permutation(vis)).cuda()
    n_pages = B * bpr
    snote = (f"bytes: the visible key pages only (the kernel also writes {score_rows * 4 / 1e6:.1f} MB "
             "of scores)")
    timed("indexer_score kernel", kbytes,
          lambda: C.indexer_score(sh, dev["q_idx"], dev["w"], keys, dev["start_pos"], bufs["scores"], stream),
          note=snote)
    timed("probe: LDS-DMA stream, address order", kbytes,
          lambda: ok(P.csa_ceiling_stream_dma(keys.data_ptr(), kbytes, d_vis.data_ptr(), n_pages,
                                              sink.data_ptr(), sptr), "dma"))
    timed("probe: LDS-DMA stream, random 16 KiB pages", kbytes,
          lambda: ok(P.csa_ceiling_stream_dma(keys.data_ptr(), kbytes, d_rand.data_ptr(), n_pages,
                                              sink.data_ptr(), sptr), "dma random"))
    timed("probe: vector-load stream, 128 KiB per workgroup", kbytes,
          lambda: ok(P.csa_ceiling_stream_vec(keys.data_ptr(), kbytes, DMA_WG_BYTES, 256, sink.data_ptr(), sptr),
                     "vec"), note="as many bytes, contiguous from the start of the key cache")

    # the same keys in a pool of 64-row (16 KiB) blocks in a seeded random
    # order: the paged score kernel, and the DMA stream reading the same
    # visible pages through the same block table
    pin = I.page_inputs({"k_idx": inp["k_idx"]}, PAGE_ROWS, seed=11, cmp=False)
    assert PAGE_ROWS == rows_per_page
    pool = torch.from_numpy(pin["k_idx_pool"].view(np.int16)).view(torch.bfloat16).cuda()
    tab = np.ascontiguousarray(pin["idx_table"], dtype=np.int32)
    table = torch.from_numpy(tab).cuda()
    pool_pages = pool.numel() * pool.element_size() // DMA_PAGE_BYTES
    assert tab.size == n_pages and 0 <= tab.min() and tab.max() < pool_pages
    d_pool_vis = torch.from_numpy(np.ascontiguousarray(tab.reshape(-1)[vis])).cuda()
    timed("indexer_score kernel, paged pool (64-row blocks)", kbytes,
          lambda: C.indexer_score_paged(sh, dev["q_idx"], dev["w"], pool, None, table, dev["start_pos"],
                                        bufs["scores"], stream), note=snote)
    timed("probe: LDS-DMA stream, the paged pool through its block table", kbytes,
          lambda: ok(P.csa_ceiling_stream_dma(pool.data_ptr(), kbytes, d_pool_vis.data_ptr(), pool_pages,
                                              sink.data_ptr(), sptr), "dma pool"))
    del pool, table, pin

    # ---- the Top-K's row read, right after the score kernel wrote the rows ---
    scores = bufs["scores"]
    sbytes = scores.numel() * scores.element_size()
    row_bytes = sh.n_cap * 4

    def score():
        C.indexer_score(sh, dev["q_idx"], dev["w"], keys, dev["start_pos"], scores, stream)

    note = "after the score kernel (untimed) wrote the rows; bytes: the whole score rows"
    timed("topk kernel", sbytes,
          lambda: C.topk(sh, scores, dev["start_pos"], bufs["topk_idx"], bufs["topk_ws"], stream),
          note=note, pre=score)
    timed("probe: read of the score rows, one 1024-thread workgroup per row", sbytes,
          lambda: ok(P.csa_ceiling_stream_vec(scores.data_ptr(), sbytes, row_bytes, 1024, sink.data_ptr(), sptr),
                     "rows"), note=note, pre=score)
    timed("probe: read of the score rows, one 256-thread workgroup per row", sbytes,
          lambda: ok(P.csa_ceiling_stream_vec(scores.data_ptr(), sbytes, row_bytes, 256, sink.data_ptr(), sptr),
                     "rows 256"), note=note, pre=score)
    timed("probe: read of the score rows, 8 256-thread workgroups per row", sbytes,
          lambda: ok(P.csa_ceiling_stream_vec(scores.data_ptr(), sbytes, row_bytes // 8, 256, sink.data_ptr(),
                                              sptr), "rows/8"), note=note, pre=score)

    # ---- the attention's row gather ----------------------------------------
    B, S, n_cap, w_cap, W = sh.batch, sh.q_per_req, sh.n_cap, sh.w_cap, sh.win
    idx = bufs["topk_idx"].cpu().numpy().reshape(B, S, -1)
    sp = inp["start_pos"].astype(np.int64)
    cmp_rows, win_rows = [], []
    for b in range(B):
        for s in range(S):
            sel = idx[b, s]
            sel = sel[(sel >= 0) & (sel < n_cap)]
            cmp_rows.append(b * n_cap + sel.astype(np.int64))
            p = sp[b] + s
            pos = np.arange(max(0, p - W + 1), p + 1)
            win_rows.append(b * w_cap + pos % w_cap)
    cmp_rows = np.concatenate(cmp_rows).astype(np.int32)
    win_rows = np.concatenate(win_rows).astype(np.int32)
    assert cmp_rows.min() >= 0 and cmp_rows.max() < B * n_cap and win_rows.max() < B * w_cap
    distinct = (np.unique(cmp_rows).size + np.unique(win_rows).size) * 2 * ROW_BYTES
    d_cmp = torch.from_numpy(cmp_rows).cuda()
    d_win = torch.from_numpy(win_rows).cuda()
    cmp_bytes = B * n_cap * ROW_BYTES
    win_bytes = B * w_cap * ROW_BYTES

    def attention():
        C.sparse_attn_decode(sh, dev["q"], dev["k_win"], dev["v_win"], dev["k_cmp"], dev["v_cmp"],
                             bufs["topk_idx"], dev["start_pos"], dev["rope_cos"], dev["rope_sin"], scale,
                             bufs["out"], bufs["attn_ws"], stream)

    def gather():
        ok(P.csa_ceiling_gather(dev["k_cmp"].data_ptr(), dev["v_cmp"].data_ptr(), cmp_bytes, d_cmp.data_ptr(),
                                int(cmp_rows.size), sink.data_ptr(), sptr), "gather cmp")
        ok(P.csa_ceiling_gather(dev["k_win"].data_ptr(), dev["v_win"].data_ptr(), win_bytes, d_win.data_ptr(),
                                int(win_rows.size), sink.data_ptr(), sptr), "gather win")

    half = (distinct // 2) // 16384 * 16384

    def sequential():
        ok(P.csa_ceiling_stream_vec(dev["k_cmp"].data_ptr(), half, 16384, 256, sink.data_ptr(), sptr), "seq k")
        ok(P.csa_ceiling_stream_vec(dev["v_cmp"].data_ptr(), half, 16384, 256, sink.data_ptr(), sptr), "seq v")

    note = "bytes: distinct K and V rows the step's lists and windows name"
    timed("attention (the library's call)", distinct, attention, note=note)
    timed("probe: K/V row gather, the same rows, 4 rows per wave (2 launches)", distinct, gather, note=note)
    timed("probe: sequential read of as many bytes (2 launches)", 2 * half, sequential)
    torch.cuda.synchronize()
    print(json.dumps({"workload": cfg.name, "device": torch.cuda.get_device_name(0), "results": results}),
          flush=True)


if __name__ == "__main__":
    main()
