"""Benchmark of one CSA sparse-attention decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--cache flushed|hot]

A step is one pass of the whole path on one batch of seeded synthetic input
already resident in HBM: indexer scoring, Top-K (with the fits-in-Top-K
bypass), and two-stream attention with the fused merge / inverse RoPE /
packing epilogue, issued through the C ABI on one stream.

Timing follows the pages' protocol of timed rounds after warm-ups ("Perf:
skip redundant CSA scoring and fuse gather unpack" and "Perf: fuse HCA merge,
inverse RoPE, and packing", descriptions): W untimed steps, then K timed
steps.  With --cache flushed (the default) a 1 GiB scratch buffer is written
and a 512 MB one read before every timed step, outside the events that
bracket the step's calls, so that neither the L2s nor the 256 MB Infinity
Cache hold anything the step reads (nor dirty lines of the flush); the step
time is the median (and minimum) of those event intervals.
A back-to-back pass of exactly K steps between two synchronisations is also
timed and reported under "hot".

Prints ONE JSON line: query tokens per second, the roofline of the dominant
kernel (algorithmic bytes / its median HIP-event-timed duration over at least
64 flushed launches, against 8 TB/s), per-stage figures, and the CPU oracle
timed on the host as a baseline.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CPU_SHARE = 16                   # host cores a one-GPU job may use on the GPU machine
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "sparse_attention_decode_csa_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3,
                    help="least number of oracle runs for the CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle runs repeat until this much CPU time has passed")
    ap.add_argument("--key-format", choices=("bf16", "fp8"), default="bf16",
                    help="indexer key cache: bf16 rows, or FP8 E4M3 codes with a per-row scale")
    ap.add_argument("--writeback", action="store_true",
                    help="start each step with the window-cache writeback of its new tokens")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK",
                    help="lay the indexer key cache and the compressed K/V cache out as pools of "
                         "BLOCK-row blocks in a seeded random order, read through block tables")
    ap.add_argument("--query-sets", type=int, default=4,
                    help="query sets cycled over the steps (queries rolled along the batch), so "
                         "consecutive steps select different compressed rows")
    ap.add_argument("--cache", choices=("flushed", "hot"), default="flushed",
                    help="flushed: 1 GiB scratch write and 512 MB clean read before each timed "
                         "step (outside its events), step time = median event interval; hot: "
                         "back-to-back steps, step time = wall time of the K steps / K")
    ap.add_argument("--stage-launches", type=int, default=64,
                    help="least number of flushed steps timed stage by stage (per-stage events)")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--no-hot", action="store_true",
                    help="skip the back-to-back pass (profiler runs of flushed launches only)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


# Source sections that the decode score kernel does not use: edits there
# leave its stored traffic counters valid.
_HASH_EXCLUDE = {"indexer_score.hip": (b"// Prefill shape:", b"hipError_t launch_gemm(")}


def kernel_source_hash(name: str, whole: bool = False) -> str:
    """Hash of the sources a kernel's stored counters were taken on (with
    whole=False, less the sections the decode kernels do not use)."""
    h = hashlib.sha256()
    for f in (name, "device_common.h"):
        text = open(os.path.join(CSRC, f), "rb").read()
        if f in _HASH_EXCLUDE and not whole:
            a, b = _HASH_EXCLUDE[f]
            i, j = text.find(a), text.find(b)
            if 0 <= i < j:
                text = text[:i] + text[j:]
        h.update(text)
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# algorithmic work: the bytes and flops the method itself must move
# --------------------------------------------------------------------------

def n_vis(p, ratio, n_cap):
    return min((p + 1) // ratio, n_cap)


def score_bytes(sh, sp, key_format="bf16"):
    """k_idx rows read once per request + scores written + q_idx + w."""
    es = 2 if sh.dtype == 1 else 4
    key_row = sh.idx_dim + 4 if key_format == "fp8" else sh.idx_dim * es   # codes + scale
    total = 0
    for b in range(sh.batch):
        nv = [n_vis(int(sp[b]) + s, sh.ratio, sh.n_cap) for s in range(sh.q_per_req)]
        scored = [n for n in nv if n > sh.topk]
        if not scored:
            continue
        total += max(scored) * key_row                  # keys, shared by the request's tokens
        total += sum(scored) * 4                        # fp32 scores
        total += sh.q_per_req * sh.idx_heads * (sh.idx_dim * es + 4)
    return total


def score_flops(sh, sp):
    f = 0
    for b in range(sh.batch):
        for s in range(sh.q_per_req):
            n = n_vis(int(sp[b]) + s, sh.ratio, sh.n_cap)
            if n > sh.topk:
                f += 2 * sh.idx_dim * sh.idx_heads * n
    return f


def topk_bytes(sh, sp):
    total = 0
    for b in range(sh.batch):
        for s in range(sh.q_per_req):
            n = n_vis(int(sp[b]) + s, sh.ratio, sh.n_cap)
            total += sh.topk * 4 + (n * 4 if n > sh.topk else 0)
    return total


def attn_bytes(sh, sp, topk_idx):
    """Distinct K+V rows per request (window union + selected union) + q + lists + out."""
    es = 2 if sh.dtype == 1 else 4
    row = 2 * sh.head_dim * es
    total = 0
    rows_attended = 0
    for b in range(sh.batch):
        win_rows, cmp_rows = set(), set()
        for s in range(sh.q_per_req):
            p = int(sp[b]) + s
            lo = max(0, p - sh.win + 1)
            win_rows.update(t % sh.w_cap for t in range(lo, p + 1))
            sel = topk_idx[b, s]
            sel = sel[(sel >= 0) & (sel < sh.n_cap)]
            cmp_rows.update(sel.tolist())
            rows_attended += (p + 1 - lo) + sel.size
        total += (len(win_rows) + len(cmp_rows)) * row
    T = sh.batch * sh.q_per_req
    total += T * sh.heads * sh.head_dim * es * 2            # q in, out
    total += T * sh.topk * 4
    return total, rows_attended


# --------------------------------------------------------------------------

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the step runs on one GPU (no multi-GPU path); run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import oracle
    from sparse_attention_decode_csa_amd import csa as C
    from sparse_attention_decode_csa_amd import inputs as I

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(3)
    C.lib()  # fail loudly if the HIP library is missing
    cfg = I.CONFIGS[args.config]
    sh = cfg.shape
    t0 = time.time()
    fp8 = args.key_format == "fp8"
    inp = I.make_inputs(args.config, key_format=args.key_format)
    t_gen = time.time() - t0
    paged = args.paged > 0
    # --paged: the indexer keys, the compressed K/V and the window rings all
    # live in block pools
    pin = I.page_inputs(inp, args.paged, seed=11, win=True) if paged else inp
    dev = C.to_device(pin, sh)
    kwin, vwin = ("k_win_pool", "v_win_pool") if paged else ("k_win", "v_win")
    bufs = C.alloc_outputs(sh)
    scale = I.softmax_scale(sh)
    stream = launch_stream = torch.cuda.current_stream()
    print(f"# config {args.config} ({cfg.name}) inputs drawn in {t_gen:.1f}s, uploaded", file=sys.stderr,
          flush=True)

    # query sets: q, q_idx and w rolled along the batch, so each request meets
    # other queries and selects other rows; caches, positions and the window
    # stay the same, as in consecutive decode steps
    R = max(1, args.query_sets)
    qsets = []
    for r in range(R):
        qs = dict(dev)
        for name in ("q", "q_idx", "w"):
            qs[name] = torch.roll(dev[name], shifts=r, dims=0).contiguous()
        qsets.append(qs)

    # window writeback: the step's new rows (as the rings already hold them, so
    # the write is idempotent) to their ring slots
    if args.writeback:
        D_ = sh.head_dim
        slots = (I.paged_ring_slot_mapping(sh, inp["start_pos"], pin["win_table"], args.paged)
                 if paged else I.ring_slot_mapping(sh, inp["start_pos"]))
        wb_slots = torch.from_numpy(slots).cuda()
        k_new = dev[kwin].reshape(-1, D_)[wb_slots.long()].contiguous()
        v_new = dev[vwin].reshape(-1, D_)[wb_slots.long()].contiguous()

    # ev: events recorded on the launch stream.  mode "step" records the two
    # that bracket the whole step (ev[0] before its first call, ev[4] after its
    # last); mode "all" also the stage boundaries: ev[1] before scoring, ev[2]
    # before Top-K, ev[3] before attention.  Each record is a packet of its own
    # in the stream, so the step timing keeps to the bracketing pair.
    def run_step(ev=None, r=0, mode="all", st=None):
        stream = st if st is not None else launch_stream
        dev = qsets[r % R]
        rec = ev is not None
        rec_all = rec and mode == "all"
        if rec: ev[0].record(stream)
        if args.writeback:
            C.swa_writeback(sh, k_new, v_new, wb_slots, dev[kwin], dev[vwin], stream)
        if rec_all: ev[1].record(stream)
        if not cfg.supplied_topk:
            if paged:
                C.indexer_score_paged(sh, dev["q_idx"], dev["w"],
                                      dev["k_idx8_pool"] if fp8 else dev["k_idx_pool"],
                                      dev["k_scale_pool"] if fp8 else None, dev["idx_table"],
                                      dev["start_pos"], bufs["scores"], stream)
            elif fp8:
                C.indexer_score_fp8(sh, dev["q_idx"], dev["w"], dev["k_idx8"], dev["k_scale"],
                                    dev["start_pos"], bufs["scores"], stream)
            else:
                C.indexer_score(sh, dev["q_idx"], dev["w"], dev["k_idx"], dev["start_pos"],
                                bufs["scores"], stream)
            if rec_all: ev[2].record(stream)
            C.topk(sh, bufs["scores"], dev["start_pos"], bufs["topk_idx"], bufs["topk_ws"], stream)
            ti = bufs["topk_idx"]
        else:
            if rec_all: ev[2].record(stream)
            ti = dev["topk_idx"]
        if rec_all: ev[3].record(stream)
        if not cfg.indexer_only and paged:
            C.sparse_attn_decode_paged(sh, dev["q"], dev[kwin], dev[vwin], dev["k_cmp_pool"],
                                       dev["v_cmp_pool"], dev["cmp_table"], ti, dev["start_pos"],
                                       dev["rope_cos"], dev["rope_sin"], scale, bufs["out"],
                                       bufs["attn_ws"], stream, win_table=dev["win_table"])
        elif not cfg.indexer_only:
            C.sparse_attn_decode(sh, dev["q"], dev["k_win"], dev["v_win"], dev["k_cmp"], dev["v_cmp"],
                                 ti, dev["start_pos"], dev["rope_cos"], dev["rope_sin"], scale,
                                 bufs["out"], bufs["attn_ws"], stream)
        if rec: ev[4].record(stream)

    # the dominant kernel: the larger algorithmic byte count (attention bytes
    # of the first query set decide it; scoring moves far more on the long
    # configurations)
    sp = inp["start_pos"]
    sb, sf = score_bytes(sh, sp, args.key_format), score_flops(sh, sp)
    run_step(r=0)
    torch.cuda.synchronize()
    ti0 = (bufs["topk_idx"] if not cfg.supplied_topk else dev["topk_idx"]).cpu().numpy()
    dominant = ("indexer_score" if cfg.indexer_only or sb >= attn_bytes(sh, sp, ti0)[0]
                else "sparse_attn")

    # Before every flushed step (outside its events): 1 GiB of scratch written,
    # more than the 256 MB Infinity Cache and the L2s together, so nothing the
    # step reads is still cached; then 512 MB of another buffer read, so that
    # the caches hold clean lines rather than the write's dirty ones, whose
    # write-back would otherwise run inside the measured kernels (measured: a
    # sequential 84 MB read takes 35 us after the write alone, 17.6 us after
    # write + read, 16.3 us with hot caches).
    scratch = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device="cuda")
    clean = torch.ones((args.flush_mib << 20) // 8, dtype=torch.float32, device="cuda")

    def flush(k):
        scratch.fill_(k & 0x7F)
        clean.sum()

    def ev_set():
        return [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    def us(e, a, b):
        return e[a].elapsed_time(e[b]) * 1e3

    for k in range(args.warmup):
        if args.cache == "flushed":
            flush(k)
        run_step(r=k)
    torch.cuda.synchronize()

    # timed region: exactly K steps between two synchronisations.  Flushed:
    # each step after a flush, bracketed by its own pair of events.  Hot: back
    # to back, wall time.  The garbage collector is held off while timing (a
    # full collection of the harness's objects stalled the launch loop for
    # tens of ms in some hot passes).
    hot_steps = args.steps
    gc.collect()
    gc.disable()
    step_us = []
    if args.cache == "flushed":
        sev = [ev_set() for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            flush(k)
            run_step(sev[k], r=k, mode="step")
        torch.cuda.synchronize()
        wall_flushed = time.perf_counter() - t0
        step_us = [us(e, 0, 4) for e in sev]
    # hot pass (the headline with --cache hot, a labelled extra otherwise)
    hot_ms = None
    if args.cache == "hot" or not args.no_hot:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(hot_steps):
            run_step(r=k)
        torch.cuda.synchronize()
        hot_ms = (time.perf_counter() - t0) * 1000.0 / hot_steps
    # the hot pass again from a HIP graph: GRAPH_STEPS steps (query set 0)
    # captured once, the graph replayed: no host launches in the loop
    graph_hot = None
    if not args.no_hot:
        GRAPH_STEPS = 10
        try:
            g = torch.cuda.CUDAGraph()
            run_step(r=0)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                for _ in range(GRAPH_STEPS):
                    run_step(r=0, st=torch.cuda.current_stream())
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, hot_steps // GRAPH_STEPS)
            t0 = time.perf_counter()
            for k in range(reps):
                g.replay()
            torch.cuda.synchronize()
            g_ms = (time.perf_counter() - t0) * 1000.0 / (reps * GRAPH_STEPS)
            graph_hot = {"cache": "hot", "ms_per_step": round(g_ms, 4),
                         "value": round(sh.batch * sh.q_per_req / (g_ms * 1e-3), 1),
                         "step_time": f"wall time of {reps} replays of a HIP graph of {GRAPH_STEPS} steps "
                                      f"/ {reps * GRAPH_STEPS}"}
            del g
        except Exception as e:  # reported, not fatal: the headline does not depend on it
            graph_hot = {"error": f"{type(e).__name__}: {e}"[:300]}
    gc.enable()
    if args.cache == "flushed":
        ms_per_step = float(np.median(step_us)) * 1e-3
    else:
        ms_per_step = hot_ms

    # stage breakdown: at least --stage-launches steps with events at every
    # stage boundary, flushed as the timed steps are (or back to back when hot)
    nb = max(args.stage_launches, min(args.steps, 300))
    gev = [ev_set() for _ in range(nb)]
    for k in range(nb):
        if args.cache == "flushed":
            flush(k)
        run_step(gev[k], r=k, mode="all")
    torch.cuda.synchronize()
    st_us = {"indexer_score": [us(e, 1, 2) for e in gev], "topk": [us(e, 2, 3) for e in gev],
             "sparse_attn": [us(e, 3, 4) for e in gev]}
    t_score = float(np.median(st_us["indexer_score"])) * 1e-6
    t_topk = float(np.median(st_us["topk"])) * 1e-6
    t_attn = float(np.median(st_us["sparse_attn"])) * 1e-6
    t_dom = float(np.median(st_us[dominant])) * 1e-6
    dom_min = float(np.min(st_us[dominant])) * 1e-6
    t_event_step = float(np.median([us(e, 0, 4) for e in gev])) * 1e-6

    tb = topk_bytes(sh, sp)
    # attention bytes depend on the selection: mean over the query sets
    abs_, rows_ = [], []
    for r in (range(R) if not cfg.indexer_only else []):
        run_step(r=r)
        torch.cuda.synchronize()
        ti = (bufs["topk_idx"] if not cfg.supplied_topk else dev["topk_idx"]).cpu().numpy()
        a_, r_ = attn_bytes(sh, sp, ti)
        abs_.append(a_)
        rows_.append(r_)
    ab, rows_att = (float(np.mean(abs_)), int(np.mean(rows_))) if abs_ else (0.0, 0)
    T = sh.batch * sh.q_per_req

    def stage(name, bytes_, t):
        gbs = bytes_ / t / 1e9 if t > 0 else 0.0
        return {"us": round(t * 1e6, 2), "us_min": round(float(np.min(st_us[name])), 2),
                "alg_bytes": int(bytes_), "GB_s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}

    stages = {"indexer_score": stage("indexer_score", sb, t_score), "topk": stage("topk", tb, t_topk),
              "sparse_attn": stage("sparse_attn", ab, t_attn)}
    stages["indexer_score"]["TFLOP_s"] = round(sf / t_score / 1e12, 2) if t_score else 0.0
    stages["sparse_attn"]["rows_attended"] = rows_att

    dom_bytes = sb if dominant == "indexer_score" else ab
    achieved = dom_bytes / t_dom / 1e9
    timing = {"kernel_us": round(t_dom * 1e6, 2), "kernel_us_min": round(dom_min * 1e6, 2),
              "kernel_launches_timed": nb, "kernel_time": "median of per-launch HIP events"}
    if cfg.indexer_only:
        # a prefill chunk re-reads each request's few MB of keys from L2 for
        # every block of query rows: the contraction, not HBM, bounds it
        roofline = dict({"bound": "mfma", "kernel": dominant}, **timing,
                        achieved=round(sf / t_dom / 1e12, 2), peak=MFMA_BF16_PEAK_TFLOPS,
                        unit="TFLOP/s", frac=round(sf / t_dom / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4))
    else:
        roofline = dict({"bound": "hbm", "kernel": dominant}, **timing, achieved=round(achieved, 1),
                        peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4))
    traffic = None
    kf = ("_fp8" if fp8 and dominant == "indexer_score" else "") + ("_paged" if paged else "")
    tfile = os.path.join(PROFILES, f"traffic_{dominant}{kf}_config{args.config}.json")
    if os.path.exists(tfile):
        tj = json.load(open(tfile))
        src = "indexer_score.hip" if dominant == "indexer_score" else "sparse_attn.hip"
        if tj.get("kernel_source_hash") == kernel_source_hash(src, whole=cfg.indexer_only):
            traffic = tj.get("hbm_bytes_per_launch")
    roofline["traffic"] = traffic

    # CPU baseline: the oracle as it stands, whole step, on the host cores this
    # job may use.  A one-GPU job's share of the host is 16 cores, whatever
    # the affinity mask shows; the counts are reported beside it.
    cpu = None
    if not args.no_cpu_baseline:
        affinity = len(os.sched_getaffinity(0))
        nthreads = max(1, min(CPU_SHARE, affinity))
        try:
            nproc = int(subprocess.run(["nproc"], capture_output=True, text=True).stdout.strip())
        except (OSError, ValueError):
            nproc = None
        times = []
        if cfg.indexer_only:   # scoring + Top-K of the chunk's first 1024 tokens
            jobs, n_tok, what = oracle.JOB_SCORE | oracle.JOB_TOPK, min(T, 1024), "scoring + Top-K"
        else:
            jobs, n_tok, what = (oracle.JOB_ATTN if cfg.supplied_topk else 7), T, "the full step"
        # at least cpu_reps runs and about cpu_seconds of oracle work in all
        # (bounded: 5000 runs, or one run past a minute)
        while len(times) < 5000:
            t0 = time.perf_counter()
            oracle.run(sh, inp, nthreads=nthreads, jobs=jobs, tokens=(0, n_tok))
            times.append(time.perf_counter() - t0)
            if times[-1] > 60 or (len(times) >= max(1, args.cpu_reps)
                                  and sum(times) >= args.cpu_seconds):
                break
        tc = float(np.median(times))
        cpu = {"value": round(n_tok / tc, 2), "unit": "query-tokens/s", "cores": nthreads,
               "kind": "oracle",
               "sample": f"{what} of {n_tok} of this workload's {T} query tokens, median of "
                         f"{len(times)} runs ({sum(times):.1f} s in all), {tc:.2f} s each, fp64 oracle",
               "nproc": nproc, "affinity_cpus": affinity,
               "hardware_concurrency": os.sysconf("SC_NPROCESSORS_ONLN"),
               "cpu_share": CPU_SHARE}
        # the long-context configuration's whole step on one thread (median of 3)
        inp3 = inp if args.config == 3 else I.make_inputs(3)
        t1 = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.run(I.CONFIGS[3].shape, inp3, nthreads=1)
            t1.append(time.perf_counter() - t0)
        del inp3
        T3 = I.CONFIGS[3].shape.batch * I.CONFIGS[3].shape.q_per_req
        cpu["long_context_1thread"] = {"s": round(float(np.median(t1)), 4),
                                       "query_tokens_per_s": round(T3 / float(np.median(t1)), 1),
                                       "sample": f"the full step of all {T3} tokens, median of 3"}

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    line = {
        "metric": ("prefill indexer query-tokens/sec (scoring + Top-K of a prefill chunk)"
                   if cfg.indexer_only else
                   "decode query-tokens/sec for CSA sparse attn step; achieved HBM GB/s vs peak"),
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == 1 else "f32",
        "data": "synthetic (seeded N(0,1) caches and queries, structure per configuration)",
        "cache": args.cache,
        "step_time": ("median of per-step HIP events bracketing the calls; before each step, "
                      "outside the events, 1 GiB of scratch written and 512 MB of another "
                      "buffer read" if args.cache == "flushed"
                      else "wall time of K back-to-back steps / K"),
        "config": {"workload": f"{cfg.name}: B={sh.batch} S={sh.q_per_req} context->"
                               f"{sh.n_cap} compressed rows (ratio {sh.ratio}) K={sh.topk} "
                               f"WIN={sh.win} H={sh.heads} D={sh.head_dim} Dr={sh.rope_dim} "
                               f"Hi={sh.idx_heads} Di={sh.idx_dim} G={sh.out_groups}",
                   "batch": sh.batch, "q_per_req": sh.q_per_req, "topk": sh.topk,
                   "max_len": sh.max_len, "query_sets": R, "indexer_keys": args.key_format,
                   "window_writeback": bool(args.writeback),
                   "paged_block_rows": args.paged or None,
                   "paged_caches": (["indexer keys", "compressed K/V", "window rings"]
                                    if paged else None),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "stages": stages,
        "stages_note": f"median (and minimum) of {nb} per-stage HIP event intervals, "
                       f"{args.cache} as the timed steps; their extra event packets add gaps, so "
                       "the stages sum above ms_per_step",
        "event_step_us": round(t_event_step * 1e6, 2),
        "hot": None if hot_ms is None else
               {"cache": "hot", "ms_per_step": round(hot_ms, 4), "value": round(T / (hot_ms * 1e-3), 1),
                "step_time": f"wall time of {hot_steps} back-to-back steps / {hot_steps}"},
        "hot_graph": graph_hot,
        "cpu_baseline": cpu,
    }
    if step_us:
        line["step_us_min"] = round(float(np.min(step_us)), 2)
        line["step_us_median"] = round(float(np.median(step_us)), 2)
        line["flushed_wall_ms_per_step"] = round(wall_flushed * 1000.0 / args.steps, 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
