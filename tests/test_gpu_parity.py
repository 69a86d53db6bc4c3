"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every expected value comes from the oracle run on the same seeded inputs.
Top-K lists must be bit-exact when both sides select from the same scores;
scores must lie within the fp32 error bound; attention outputs within max-abs
2e-2 (bf16) or 1e-5 row-relative (fp32).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_csa_amd import csa as C
from sparse_attention_decode_csa_amd import inputs as I
from tests import _util as U

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    C.lib()
    yield
    torch.cuda.synchronize()


def small_cfg(name="edge", seed=21, structure="none", lengths=None, **kw):
    base = dict(batch=4, q_per_req=2, ratio=4, n_cap=256, topk=64, win=64, w_cap=96, heads=16,
                head_dim=128, rope_dim=64, idx_heads=4, idx_dim=128, out_groups=1, max_len=1024,
                dtype=I.BF16)
    base.update(kw)
    sh = I.Shape(**base)
    return I.Config(name=name, shape=sh, seed=seed,
                    lengths=lengths or f"start_uniform:0:{sh.max_len - sh.q_per_req}",
                    structure=structure, supplied_topk=False)


def gpu_step(shape, inp, supplied=False, topk_idx=None, scores=None, jobs=("score", "topk", "attn")):
    """Run chosen steps on the GPU; returns numpy copies of scores, topk_idx, out."""
    d = C.to_device(inp, shape)
    bufs = C.alloc_outputs(shape)
    scale = I.softmax_scale(shape)
    if scores is not None:
        bufs["scores"].copy_(torch.from_numpy(scores))
    if "score" in jobs:
        if "idx_table" in d:   # paged indexer key cache
            fp8 = "k_idx8_pool" in d
            C.indexer_score_paged(shape, d["q_idx"], d["w"], d["k_idx8_pool" if fp8 else "k_idx_pool"],
                                  d["k_scale_pool"] if fp8 else None, d["idx_table"],
                                  d["start_pos"], bufs["scores"])
        elif "k_idx8" in d:   # FP8 indexer key cache
            C.indexer_score_fp8(shape, d["q_idx"], d["w"], d["k_idx8"], d["k_scale"], d["start_pos"],
                                bufs["scores"])
        else:
            C.indexer_score(shape, d["q_idx"], d["w"], d["k_idx"], d["start_pos"], bufs["scores"])
    if "topk" in jobs:
        C.topk(shape, bufs["scores"], d["start_pos"], bufs["topk_idx"], bufs["topk_ws"])
    ti = bufs["topk_idx"]
    if topk_idx is not None:
        ti = torch.from_numpy(np.ascontiguousarray(topk_idx, np.int32)).cuda()
    elif supplied:
        ti = d["topk_idx"]
    if "attn" in jobs and "cmp_table" in d:   # paged compressed K/V cache (window maybe paged)
        pw = "win_table" in d
        C.sparse_attn_decode_paged(shape, d["q"], d["k_win_pool" if pw else "k_win"],
                                   d["v_win_pool" if pw else "v_win"], d["k_cmp_pool"],
                                   d["v_cmp_pool"], d["cmp_table"], ti, d["start_pos"],
                                   d["rope_cos"], d["rope_sin"], scale, bufs["out"], bufs["attn_ws"],
                                   win_table=d.get("win_table"))
    elif "attn" in jobs:
        C.sparse_attn_decode(shape, d["q"], d["k_win"], d["v_win"], d["k_cmp"], d["v_cmp"], ti,
                             d["start_pos"], d["rope_cos"], d["rope_sin"], scale, bufs["out"],
                             bufs["attn_ws"])
    torch.cuda.synchronize()
    return dict(scores=bufs["scores"].cpu().numpy(), topk_idx=bufs["topk_idx"].cpu().numpy(),
                out=bufs["out"].float().cpu().numpy())


def oracle_step(cfg_shape, inp, **kw):
    return oracle.run(cfg_shape, inp, nthreads=NTHREADS, **kw)


# --------------------------------------------------------------------------
# attention on the oracle's own Top-K lists
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cid", [0, 1, 2])
def test_attention_matches_oracle(cid, config_inputs):
    cfg = I.CONFIGS[cid]
    sh, inp = cfg.shape, config_inputs(cid)
    ref = oracle_step(sh, inp, jobs=(oracle.JOB_ATTN if cfg.supplied_topk
                                     else oracle.JOB_SCORE | oracle.JOB_TOPK | oracle.JOB_ATTN))
    got = gpu_step(sh, inp, topk_idx=ref["topk_idx"], jobs=("attn",))
    worst = U.compare_outputs(sh, got["out"], ref["out"])
    print(f"config {cid}: worst error {worst:.3g}")


# Shapes on either side of the one-workgroup-per-token kernel: window and
# Top-K rows within 12 waves of at most 4 chunks of 16 rows, at most 4096
# tokens and at least 384 waves in all take it (no workspace); the rest take
# the split kernels (4, 2 or 1 chunks per wave).  Random lists of visible rows with duplicates, padding and
# out-of-range entries; the output must match the oracle and repeat bit for
# bit.
ATTN_PATHS = [
    # split kernels
    (dict(batch=2, q_per_req=1, win=64, w_cap=64, topk=1024), True),                       # 1 chunk/wave
    (dict(batch=3, q_per_req=4, win=128, w_cap=131, topk=1024, heads=8, out_groups=2), True),   # 2
    (dict(batch=32, q_per_req=4, win=256, w_cap=259, topk=800, head_dim=64, rope_dim=32,
          out_groups=4), True),                                                          # 4
    (dict(batch=8, q_per_req=8, win=96, w_cap=103, topk=1024, heads=4, head_dim=64, rope_dim=0,
          dtype=I.F32, idx_dim=64), True),
    (dict(batch=3, q_per_req=1, win=100, w_cap=100, topk=200, rope_dim=2, dtype=I.F32), True),
    (dict(batch=4100, q_per_req=1, n_cap=64, max_len=256, win=16, w_cap=16, topk=16, heads=2,
          head_dim=64, rope_dim=64, idx_heads=1, idx_dim=64), True),                       # tokens
    # more than 16 query heads: one split workgroup per group of 16 heads
    (dict(batch=4, q_per_req=2, heads=64, out_groups=4, win=64, w_cap=65, topk=256), True),
    (dict(batch=3, q_per_req=1, heads=20, out_groups=5, head_dim=64, rope_dim=32, win=100,
          w_cap=100, topk=300), True),
    (dict(batch=2, q_per_req=3, heads=48, out_groups=3, dtype=I.F32, win=40, w_cap=42, topk=128),
     True),
    (dict(batch=2, q_per_req=2, heads=32, head_dim=64, rope_dim=0, dtype=I.F32, win=64, w_cap=65,
          topk=64, idx_dim=64), True),
    (dict(batch=4, q_per_req=2, win=128, w_cap=129, topk=512), True),   # 4 chunks, 80 waves
    (dict(batch=3, q_per_req=3, win=32, w_cap=34, topk=100, heads=5, head_dim=64), True),  # 81 waves
    # one workgroup per token
    (dict(batch=128, q_per_req=2, win=128, w_cap=129, topk=512), False),                   # 4 chunks
    (dict(batch=256, q_per_req=1, win=64, w_cap=64, topk=256, out_groups=2), False),       # 2
    (dict(batch=40, q_per_req=3, win=32, w_cap=34, topk=100, heads=5, head_dim=64), False),  # 1
    (dict(batch=48, q_per_req=2, win=64, w_cap=65, topk=100, rope_dim=32, out_groups=4,
          dtype=I.F32), False),
    (dict(batch=64, q_per_req=4, win=200, w_cap=203, topk=300, heads=3, head_dim=64, rope_dim=16,
          out_groups=3, dtype=I.F32, idx_dim=64), False),
]


@pytest.mark.parametrize("case", range(len(ATTN_PATHS)))
def test_attention_split_and_token_paths(case):
    kw, split = ATTN_PATHS[case]
    cfg = small_cfg(name="paths", seed=40 + case, **kw)
    sh = cfg.shape
    assert (C.sparse_attn_workspace_bytes(sh) > 0) == split
    inp = I.make_inputs(cfg)
    g = np.random.default_rng(400 + case)
    B, S, K = sh.batch, sh.q_per_req, sh.topk
    p = inp["start_pos"].astype(np.int64)[:, None] + np.arange(S)[None, :]
    nv = np.minimum((p + 1) // sh.ratio, sh.n_cap)[..., None]
    ti = (g.random((B, S, K)) * nv).astype(np.int32)            # visible rows, repeats allowed
    pad = (g.random((B, S, K)) < 0.1) | (nv == 0)
    ti = np.where(pad, g.choice(np.int32([-3, -1, sh.n_cap, sh.n_cap + 2]), size=(B, S, K)), ti)
    ref = oracle_step(sh, inp, jobs=oracle.JOB_ATTN, topk_idx=ti)
    got = gpu_step(sh, inp, topk_idx=ti, jobs=("attn",))
    worst = U.compare_outputs(sh, got["out"], ref["out"])
    again = gpu_step(sh, inp, topk_idx=ti, jobs=("attn",))
    assert np.array_equal(got["out"], again["out"])
    print(f"case {case} ({'split' if split else 'token'}): worst error {worst:.3g}")


# --------------------------------------------------------------------------
# indexer scores
# --------------------------------------------------------------------------

def check_scores(sh, inp, got, ref):
    rows = U.token_rows(sh, inp["start_pos"])
    bound = U.score_error_bound(sh, inp, rows)
    assert rows, "configuration scores nothing"
    scored = np.zeros(got["scores"].shape, dtype=bool)
    for (b, s, n) in rows:
        err = np.abs(got["scores"][b, s, :n].astype(np.float64) - ref["scores"][b, s, :n])
        assert np.all(err <= bound[(b, s)]), f"token {(b, s)}: score error above bound"
        scored[b, s, :n] = True
    assert np.isnan(got["scores"][~scored]).all(), "entries outside the scored set were written"


@pytest.mark.parametrize("cid", [0, 3])
def test_scores_match_oracle(cid, config_inputs):
    cfg = I.CONFIGS[cid]
    sh, inp = cfg.shape, config_inputs(cid)
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE)
    got = gpu_step(sh, inp, jobs=("score",))
    rows = U.token_rows(sh, inp["start_pos"])
    bound = U.score_error_bound(sh, inp, rows)
    assert rows, "configuration scores nothing"
    scored = np.zeros(got["scores"].shape, dtype=bool)
    for (b, s, n) in rows:
        err = np.abs(got["scores"][b, s, :n].astype(np.float64) - ref["scores"][b, s, :n])
        assert np.all(err <= bound[(b, s)]), f"token {(b, s)}: score error above bound"
        scored[b, s, :n] = True
    assert np.isnan(got["scores"][~scored]).all(), "entries outside the scored set were written"


@pytest.mark.parametrize("S,Hi,Di", [(1, 4, 128), (2, 8, 128), (4, 8, 64), (8, 8, 128), (3, 5, 64)])
def test_scores_exact_grid(S, Hi, Di):
    # Dyadic-grid inputs make every fp32 partial sum exact: bitwise equality.
    cfg = small_cfg(q_per_req=S, idx_heads=Hi, idx_dim=Di, n_cap=600, topk=32, max_len=2400)
    inp = I.make_inputs(cfg)
    g = np.random.default_rng(S * 100 + Hi)
    inp["q_idx"] = I.f32_to_bf16_bits((g.integers(-8, 9, inp["q_idx"].shape) / 4.0).astype(np.float32))
    kg = I.f32_to_bf16_bits((g.integers(-8, 9, inp["k_idx"].shape) / 4.0).astype(np.float32))
    inp["k_idx"] = np.where(inp["k_idx"] == I.f32_to_bf16_bits(np.float32([I.POISON]))[0],
                            inp["k_idx"], kg)
    inp["w"] = (g.integers(0, 17, inp["w"].shape) / 16.0).astype(np.float32)
    sh = cfg.shape
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE)
    got = gpu_step(sh, inp, jobs=("score",))
    assert np.array_equal(got["scores"], ref["scores"], equal_nan=True)


# --------------------------------------------------------------------------
# FP8 indexer key cache (E4M3 codes + per-row scale)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cid", [3, 4])
def test_scores_fp8_match_oracle(cid):
    sh = I.CONFIGS[cid].shape
    inp = I.make_inputs(cid, key_format="fp8")
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE)
    got = gpu_step(sh, inp, jobs=("score",))
    check_scores(sh, inp, got, ref)


@pytest.mark.parametrize("S,Hi,Di", [(1, 4, 128), (2, 8, 128), (4, 8, 64), (8, 8, 128), (3, 5, 64),
                                     (2, 16, 128)])
def test_scores_fp8_exact_grid(S, Hi, Di):
    # Keys on the dyadic grid are exact E4M3 codes; with power-of-two scales
    # every partial sum is exact on both sides: bitwise equality.
    cfg = small_cfg(q_per_req=S, idx_heads=Hi, idx_dim=Di, n_cap=600, topk=32, max_len=2400)
    inp = I.make_inputs(cfg, key_format="fp8")
    g = np.random.default_rng(S * 1000 + Hi * 10 + Di)
    inp["q_idx"] = I.f32_to_bf16_bits((g.integers(-8, 9, inp["q_idx"].shape) / 4.0).astype(np.float32))
    inp["w"] = (g.integers(0, 17, inp["w"].shape) / 16.0).astype(np.float32)
    live = inp["k_scale"] < 1.0   # rows quantised from N(0,1) keys; poisoned rows keep theirs
    codes = I.f32_to_e4m3_bits((g.integers(-8, 9, inp["k_idx8"].shape) / 4.0).astype(np.float32))
    inp["k_idx8"] = np.where(live[..., None], codes, inp["k_idx8"])
    pow2 = np.exp2(g.integers(-1, 2, inp["k_scale"].shape)).astype(np.float32)
    inp["k_scale"] = np.where(live, pow2, inp["k_scale"]).astype(np.float32)
    sh = cfg.shape
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE)
    got = gpu_step(sh, inp, jobs=("score",))
    assert np.array_equal(got["scores"], ref["scores"], equal_nan=True)


def test_end_to_end_fp8_keys():
    # FP8 scoring, GPU Top-K and attention on the wide Top-K configuration
    cid = 4
    sh = I.CONFIGS[cid].shape
    inp = I.make_inputs(cid, key_format="fp8")
    ref = oracle_step(sh, inp)
    got = gpu_step(sh, inp)
    rows = U.token_rows(sh, inp["start_pos"])
    bound = U.score_error_bound(sh, inp, rows)
    exempt = U.topk_exemptions(sh, got["topk_idx"], ref["topk_idx"], ref["scores"], bound,
                               inp["start_pos"])
    print(f"fp8 config {cid}: {len(exempt)} boundary exemptions {exempt}")
    assert len(exempt) <= max(1, sh.batch * sh.q_per_req // 32)
    ex = {b * sh.q_per_req + s for (b, s, _) in exempt}
    keep = [t for t in range(sh.batch * sh.q_per_req) if t not in ex]
    U.compare_outputs(sh, got["out"], ref["out"], tokens=keep)


# --------------------------------------------------------------------------
# paged compressed caches: pools of blocks located through block tables
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cid,bs,fmt", [(3, 16, "bf16"), (3, 256, "fp8"), (4, 64, "bf16"),
                                        (4, 4096, "fp8"), (0, 16, "bf16")])
def test_paged_scores_match_oracle(cid, bs, fmt):
    sh = I.CONFIGS[cid].shape
    dense = I.make_inputs(cid, key_format=fmt)
    inp = I.page_inputs(dense, bs, seed=cid * 10 + bs, cmp=False)
    ref = oracle.run_paged(sh, inp, jobs=oracle.JOB_SCORE, nthreads=NTHREADS)
    got = gpu_step(sh, inp, jobs=("score",))
    check_scores(sh, dense, got, ref)
    # the paged kernel does the dense kernel's arithmetic in the same order
    assert np.array_equal(got["scores"], gpu_step(sh, dense, jobs=("score",))["scores"],
                          equal_nan=True)


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_paged_scores_exact_grid_ragged(fmt):
    # n_cap not a multiple of the block size, spare table columns pointing
    # at poisoned blocks, dyadic inputs: bitwise equality with the oracle.
    cfg = small_cfg(q_per_req=3, idx_heads=8, idx_dim=128, n_cap=600, topk=32, max_len=2400)
    inp = I.make_inputs(cfg, key_format=fmt)
    g = np.random.default_rng(77)
    inp["q_idx"] = I.f32_to_bf16_bits((g.integers(-8, 9, inp["q_idx"].shape) / 4.0).astype(np.float32))
    inp["w"] = (g.integers(0, 17, inp["w"].shape) / 16.0).astype(np.float32)
    if fmt == "fp8":
        live = inp["k_scale"] < 1.0
        codes = I.f32_to_e4m3_bits((g.integers(-8, 9, inp["k_idx8"].shape) / 4.0).astype(np.float32))
        inp["k_idx8"] = np.where(live[..., None], codes, inp["k_idx8"])
    else:
        kg = I.f32_to_bf16_bits((g.integers(-8, 9, inp["k_idx"].shape) / 4.0).astype(np.float32))
        inp["k_idx"] = np.where(inp["k_idx"] == I.f32_to_bf16_bits(np.float32([I.POISON]))[0],
                                inp["k_idx"], kg)
    paged = I.page_inputs(inp, 64, seed=5, cmp=False)
    t = paged["idx_table"]
    spare = np.setdiff1d(np.arange(paged["k_idx8_pool" if fmt == "fp8" else "k_idx_pool"].shape[0]),
                         t.reshape(-1)).astype(np.int32)
    paged["idx_table"] = np.concatenate([t, np.tile(spare[:1], (t.shape[0], 7))], axis=1)
    sh = cfg.shape
    ref = oracle.run_paged(sh, paged, jobs=oracle.JOB_SCORE, nthreads=NTHREADS)
    got = gpu_step(sh, paged, jobs=("score",))
    assert np.array_equal(got["scores"], ref["scores"], equal_nan=True)


@pytest.mark.parametrize("cid,bs,win", [(0, 16, False), (1, 32, False), (2, 16, False), (4, 128, False),
                                        (0, 16, True), (2, 16, True), (3, 32, True), (4, 64, True)])
def test_paged_attention_matches_oracle(cid, bs, win):
    # compressed K/V paged, and with win=True the window rings too
    cfg = I.CONFIGS[cid]
    sh = cfg.shape
    dense = I.make_inputs(cid)
    inp = I.page_inputs(dense, bs, seed=cid + 40, idx=False, win=win)
    ref = oracle.run_paged(sh, inp, nthreads=NTHREADS,
                           jobs=(oracle.JOB_ATTN if cfg.supplied_topk
                                 else oracle.JOB_SCORE | oracle.JOB_TOPK | oracle.JOB_ATTN))
    got = gpu_step(sh, inp, topk_idx=ref["topk_idx"], jobs=("attn",))
    worst = U.compare_outputs(sh, got["out"], ref["out"])
    print(f"paged config {cid} block {bs} window paged {win}: worst error {worst:.3g}")
    # same rows in the same order as the dense path: identical outputs
    dgot = gpu_step(sh, dense, topk_idx=ref["topk_idx"], jobs=("attn",))
    assert np.array_equal(got["out"], dgot["out"])


@pytest.mark.parametrize("fmt,bs,win", [("bf16", 64, True), ("fp8", 16, False)])
def test_end_to_end_paged(fmt, bs, win):
    # score, select and attend with the indexer and compressed caches paged
    # (and the window rings with win=True), on the wide Top-K configuration,
    # against the oracle over the gathered caches
    cid = 4
    sh = I.CONFIGS[cid].shape
    dense = I.make_inputs(cid, key_format=fmt)
    inp = I.page_inputs(dense, bs, seed=9, win=win)
    ref = oracle.run_paged(sh, inp, nthreads=NTHREADS)
    got = gpu_step(sh, inp)
    rows = U.token_rows(sh, inp["start_pos"])
    bound = U.score_error_bound(sh, dense, rows)
    exempt = U.topk_exemptions(sh, got["topk_idx"], ref["topk_idx"], ref["scores"], bound,
                               inp["start_pos"])
    print(f"paged {fmt} block {bs}: {len(exempt)} boundary exemptions {exempt}")
    assert len(exempt) <= max(1, sh.batch * sh.q_per_req // 32)
    ex = {b * sh.q_per_req + s for (b, s, _) in exempt}
    keep = [t for t in range(sh.batch * sh.q_per_req) if t not in ex]
    U.compare_outputs(sh, got["out"], ref["out"], tokens=keep)


@pytest.mark.parametrize("heads,groups,bs", [(64, 4, 32), (32, 1, 16)])
def test_end_to_end_paged_many_heads(heads, groups, bs):
    # the whole step with 32 or 64 query heads (split workgroups per group of
    # 16 heads) over paged caches, against the oracle over the gathered caches
    cfg = small_cfg(name="heads", seed=31 + heads, batch=4, q_per_req=2, heads=heads,
                    out_groups=groups, n_cap=512, max_len=2048, topk=128, win=64, w_cap=80,
                    lengths="start_uniform:800:2046")
    sh = cfg.shape
    dense = I.make_inputs(cfg)
    inp = I.page_inputs(dense, bs, seed=heads, win=True)
    ref = oracle.run_paged(sh, inp, nthreads=NTHREADS)
    got = gpu_step(sh, inp)
    rows = U.token_rows(sh, inp["start_pos"])
    bound = U.score_error_bound(sh, dense, rows)
    exempt = U.topk_exemptions(sh, got["topk_idx"], ref["topk_idx"], ref["scores"], bound,
                               inp["start_pos"])
    assert len(exempt) <= 1, exempt
    ex = {b * sh.q_per_req + s for (b, s, _) in exempt}
    keep = [t for t in range(sh.batch * sh.q_per_req) if t not in ex]
    U.compare_outputs(sh, got["out"], ref["out"], tokens=keep)


# --------------------------------------------------------------------------
# prefill indexer: many query tokens per request (q_per_req = chunk length)
# --------------------------------------------------------------------------

def prefill_cfg(T, K, Hi, start, B=2, grid=False, Di=128, key_format="bf16"):
    max_len = start + T
    cfg = small_cfg(name="prefill", batch=B, q_per_req=T, topk=K, idx_heads=Hi, idx_dim=Di,
                    n_cap=max(256, max_len // 4), win=64, w_cap=64 + T, heads=4,
                    max_len=max_len)
    inp = I.make_inputs(cfg, start_pos=np.full(B, start, np.int32), key_format=key_format)
    if grid:   # dyadic grid: every partial sum exact on both sides
        g = np.random.default_rng(T + K)
        inp["q_idx"] = I.f32_to_bf16_bits((g.integers(-8, 9, inp["q_idx"].shape) / 4.0).astype(np.float32))
        kg = I.f32_to_bf16_bits((g.integers(-8, 9, inp["k_idx"].shape) / 4.0).astype(np.float32))
        inp["k_idx"] = np.where(inp["k_idx"] == I.f32_to_bf16_bits(np.float32([I.POISON]))[0],
                                inp["k_idx"], kg)
        inp["w"] = (g.integers(0, 17, inp["w"].shape) / 16.0).astype(np.float32)
    return cfg.shape, inp


@pytest.mark.parametrize("T,K,Hi,start,fmt", [(512, 64, 8, 0, "bf16"), (1024, 256, 8, 3000, "bf16"),
                                              (300, 128, 5, 1000, "bf16"), (2048, 1024, 4, 30000, "bf16"),
                                              (1024, 512, 8, 12000, "fp8"), (600, 128, 16, 4000, "fp8")])
def test_prefill_indexer_topk(T, K, Hi, start, fmt):
    # Each of the T tokens scores its own causally visible rows (widths well
    # past 256) and selects its own Top-K; bypass tokens get bounded indices.
    # fp8: an FP8 key cache with per-row amax/448 scales (GEMM-shaped kernel).
    sh, inp = prefill_cfg(T, K, Hi, start, key_format=fmt)
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE | oracle.JOB_TOPK)
    got = gpu_step(sh, inp, jobs=("score", "topk"))
    check_scores(sh, inp, got, ref)
    rows = U.token_rows(sh, inp["start_pos"])
    bound = U.score_error_bound(sh, inp, rows)
    exempt = U.topk_exemptions(sh, got["topk_idx"], ref["topk_idx"], ref["scores"], bound,
                               inp["start_pos"])
    print(f"prefill {fmt} T={T}: {len(rows)} scored tokens, {len(exempt)} boundary exemptions")
    assert len(exempt) <= max(1, len(rows) // 32)
    # and the selection alone is bit-exact on the oracle's scores
    got2 = gpu_step(sh, inp, scores=ref["scores"], jobs=("topk",))
    assert np.array_equal(got2["topk_idx"], ref["topk_idx"])


@pytest.mark.parametrize("T,K,Hi,start,Di,bs", [
    (600, 256, 8, 1500, 128, 0),      # partial last row block and key step
    (533, 100, 4, 5000, 64, 0),
    (200, 64, 16, 9000, 128, 0),
    (700, 512, 8, 9300, 128, 0),      # several key blocks of 1024
    (600, 256, 8, 1500, 128, 16),     # paged indexer cache
    (533, 100, 4, 5000, 64, 64),
    (300, 150, 8, 500, 128, 0),       # blocks mixing tokens that fit Top-K with scored ones
])
def test_prefill_indexer_exact_grid(T, K, Hi, start, Di, bs):
    # Dyadic inputs: every partial sum is exact on both sides, so scores and
    # lists are bitwise equal.  Chunks of at least 2048 query rows per request
    # with 4, 8 or 16 heads take the shared-key-step score kernel.
    sh, inp = prefill_cfg(T, K, Hi, start, grid=True, Di=Di)
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE | oracle.JOB_TOPK)
    if bs:
        inp = I.page_inputs(inp, bs, seed=T + bs, cmp=False)
    got = gpu_step(sh, inp, jobs=("score", "topk"))
    assert np.array_equal(got["scores"], ref["scores"], equal_nan=True)
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])


@pytest.mark.parametrize("T,K,Hi,start,Di,bs,scales", [
    (600, 256, 8, 1500, 128, 0, "pow2"),     # GEMM-shaped kernel, FP8 keys
    (333, 100, 4, 5000, 64, 16, "pow2"),     # 64 dims: decode-shaped kernel, paged codes and scales
    (300, 64, 16, 9000, 128, 0, "one"),
    (300, 150, 5, 500, 64, 0, "pow2"),       # 5 heads: the LDS head-sum path; tokens that fit Top-K
    (700, 256, 8, 3000, 128, 64, "pow2"),    # GEMM-shaped, paged (64-row blocks)
    (1100, 128, 4, 2000, 128, 16, "pow2"),   # GEMM-shaped, paged (16-row blocks), 4 heads
    (1100, 512, 8, 12000, 128, 0, "pow2"),   # several key blocks and row blocks
])
def test_prefill_indexer_fp8_exact_grid(T, K, Hi, start, Di, bs, scales):
    # A prefill chunk over an FP8 indexer key cache: the grid keys m/4 are
    # E4M3 values, so codes hold them exactly; row scales that are powers of
    # two keep every product exact, so scores and lists stay bitwise equal.
    # Chunks of at least 4096 query rows per request with 128-dim keys and 4,
    # 8 or 16 heads run the GEMM-shaped kernel, the others the decode-shaped
    # one; the scales are drawn per row, so that a scale applied to the wrong
    # key shows.
    sh, inp = prefill_cfg(T, K, Hi, start, grid=True, Di=Di)
    kf = I.bf16_bits_to_f32(inp.pop("k_idx"))
    inp["k_idx8"] = I.f32_to_e4m3_bits(kf)          # poison saturates to 448: never read
    if scales == "one":
        inp["k_scale"] = np.ones(kf.shape[:2], dtype=np.float32)
    else:
        g = np.random.default_rng(T * 7 + Hi)
        inp["k_scale"] = np.exp2(g.integers(-2, 3, size=kf.shape[:2])).astype(np.float32)
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE | oracle.JOB_TOPK)
    if bs:
        inp = I.page_inputs(inp, bs, seed=T + bs, cmp=False)
    got = gpu_step(sh, inp, jobs=("score", "topk"))
    assert np.array_equal(got["scores"], ref["scores"], equal_nan=True)
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])


# --------------------------------------------------------------------------
# window-cache writeback
# --------------------------------------------------------------------------

def to_gpu(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


@pytest.mark.parametrize("B,S,D,dt", [(1, 1, 128, I.BF16), (31, 1, 128, I.BF16), (11, 3, 64, I.BF16),
                                      (257, 16, 128, I.BF16), (127, 1, 64, I.F32)])
def test_writeback_matches_oracle(B, S, D, dt):
    # token counts 1, 31, 33, 4112 and 127: no tile multiple; some slots padding
    g = np.random.default_rng(B * 100 + S)
    T, n_slots = B * S, B * S * 2 + 7
    npdt = np.uint16 if dt == I.BF16 else np.float32
    if dt == I.BF16:
        cache = g.integers(0, 2 ** 16, size=(2, n_slots, D)).astype(np.uint16)
        new = g.integers(0, 2 ** 16, size=(2, T, D)).astype(np.uint16)
    else:
        cache = g.standard_normal(size=(2, n_slots, D)).astype(npdt)
        new = g.standard_normal(size=(2, T, D)).astype(npdt)
    slots = g.permutation(n_slots)[:T].astype(np.int32)
    pad = g.random(T) < 0.1
    slots[pad] = np.where(g.random(int(pad.sum())) < 0.5, -3, n_slots)
    ref_k, ref_v = oracle.swa_writeback(new[0], new[1], slots, cache[0], cache[1])
    sh = small_cfg(batch=B, q_per_req=S, head_dim=D, dtype=dt).shape
    kc, vc = to_gpu(cache[0]), to_gpu(cache[1])
    C.swa_writeback(sh, to_gpu(new[0]), to_gpu(new[1]), to_gpu(slots), kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), ref_k) and np.array_equal(vc.cpu().numpy(), ref_v)


def test_writeback_then_attention():
    # the step's new window entries start poisoned in the rings; the GPU
    # writeback through the ring mapping must restore the oracle's output
    cfg = small_cfg(batch=4, q_per_req=3, win=48, w_cap=53, max_len=1024)
    sh = cfg.shape
    inp = I.make_inputs(cfg)
    ref = oracle_step(sh, inp)
    B, S, Wc, D = sh.batch, sh.q_per_req, sh.w_cap, sh.head_dim
    slots = I.ring_slot_mapping(sh, inp["start_pos"])
    kflat = inp["k_win"].reshape(B * Wc, D)
    vflat = inp["v_win"].reshape(B * Wc, D)
    k_new, v_new = kflat[slots].copy(), vflat[slots].copy()
    poison = I.f32_to_bf16_bits(np.float32([I.POISON]))[0]
    kp, vp = kflat.copy(), vflat.copy()
    kp[slots] = poison
    vp[slots] = poison
    d = C.to_device(dict(inp, k_win=kp.reshape(B, Wc, D), v_win=vp.reshape(B, Wc, D)), sh)
    bufs = C.alloc_outputs(sh)
    C.swa_writeback(sh, C.to_device(dict(x=k_new), sh)["x"], C.to_device(dict(x=v_new), sh)["x"],
                    to_gpu(slots), d["k_win"], d["v_win"])
    ti = to_gpu(ref["topk_idx"])   # the oracle's lists: this checks the window alone
    C.sparse_attn_decode(sh, d["q"], d["k_win"], d["v_win"], d["k_cmp"], d["v_cmp"], ti,
                         d["start_pos"], d["rope_cos"], d["rope_sin"], I.softmax_scale(sh),
                         bufs["out"], bufs["attn_ws"])
    torch.cuda.synchronize()
    U.compare_outputs(sh, bufs["out"].float().cpu().numpy(), ref["out"])


@pytest.mark.parametrize("bs", [16, 32])
def test_writeback_then_attention_paged_window(bs):
    # the window rings live in a pool; the step's new entries start poisoned
    # there, the GPU writeback through the paged slot mapping restores them and
    # the paged attention must then give the oracle's output
    cfg = small_cfg(batch=4, q_per_req=3, win=48, w_cap=53, max_len=1024)
    sh = cfg.shape
    dense = I.make_inputs(cfg)
    ref = oracle_step(sh, dense)
    inp = I.page_inputs(dense, bs, seed=21, idx=False, win=True)
    D = sh.head_dim
    slots = I.paged_ring_slot_mapping(sh, dense["start_pos"], inp["win_table"], bs)
    kflat = inp["k_win_pool"].reshape(-1, D)
    vflat = inp["v_win_pool"].reshape(-1, D)
    k_new, v_new = kflat[slots].copy(), vflat[slots].copy()
    poison = I.f32_to_bf16_bits(np.float32([I.POISON]))[0]
    kp, vp = kflat.copy(), vflat.copy()
    kp[slots] = poison
    vp[slots] = poison
    d = C.to_device(dict(inp, k_win_pool=kp.reshape(inp["k_win_pool"].shape),
                         v_win_pool=vp.reshape(inp["v_win_pool"].shape)), sh)
    bufs = C.alloc_outputs(sh)
    C.swa_writeback(sh, C.to_device(dict(x=k_new), sh)["x"], C.to_device(dict(x=v_new), sh)["x"],
                    to_gpu(slots), d["k_win_pool"], d["v_win_pool"])
    ti = to_gpu(ref["topk_idx"])
    C.sparse_attn_decode_paged(sh, d["q"], d["k_win_pool"], d["v_win_pool"], d["k_cmp_pool"],
                               d["v_cmp_pool"], d["cmp_table"], ti, d["start_pos"], d["rope_cos"],
                               d["rope_sin"], I.softmax_scale(sh), bufs["out"], bufs["attn_ws"],
                               win_table=d["win_table"])
    torch.cuda.synchronize()
    U.compare_outputs(sh, bufs["out"].float().cpu().numpy(), ref["out"])


# --------------------------------------------------------------------------
# Top-K: bit-exact on the same scores
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cid", [0, 3, 4])
def test_topk_exact_on_oracle_scores(cid, config_inputs):
    cfg = I.CONFIGS[cid]
    sh, inp = cfg.shape, config_inputs(cid)
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE | oracle.JOB_TOPK)
    got = gpu_step(sh, inp, scores=ref["scores"], jobs=("topk",))
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])


@pytest.mark.parametrize("kind", ["normal", "coarse", "signed_zero", "spiked16", "spiked32"])
@pytest.mark.parametrize("n_cap,topk", [(300, 64), (4096, 256), (4096, 257), (9000, 1024),
                                        (16384, 512), (32768, 1024), (32768, 4096), (40000, 2048),
                                        (1000, 999), (20000, 4000), (4100, 1024), (12292, 2048),
                                        (65536, 1024), (131072, 512), (131072, 64)])
def test_topk_exact_synthetic(kind, n_cap, topk):
    # "spiked" rows put their largest values exactly where the selection's
    # strided sample looks, so the sampled threshold keeps too few rows and
    # the full-row selection must take over; "coarse" rows tie heavily.
    # rows of several visible lengths, including n_vis == K and K + 1.
    # 4100 and 12292 are multiples of 4 but not of the per-thread slice length
    # (8 and 16), so a thread's slice would straddle n_cap: the selection must
    # take its per-element load path there.  Rows past 32768 keys take the
    # two-pass selection (chunks, then a merge), short rows of the same launch
    # included.
    B, S = 3, 2
    sh = I.Shape(batch=B, q_per_req=S, ratio=4, n_cap=n_cap, topk=topk, win=8, w_cap=16, heads=1,
                 head_dim=64, rope_dim=0, idx_heads=1, idx_dim=64, out_groups=1,
                 max_len=4 * n_cap, dtype=I.BF16)
    sp = np.array([4 * n_cap - S, 4 * topk - 1, 4 * (topk + 1) - 1 - 1], np.int32)
    sp = np.minimum(sp, 4 * n_cap - S).astype(np.int32)
    scores = I.random_scores(n_cap + topk, B, S, n_cap, kind)
    inp = dict(start_pos=sp)
    ref = oracle.run(sh, inp, jobs=oracle.JOB_TOPK, scores=scores)
    d_scores = torch.from_numpy(scores).cuda()
    d_sp = torch.from_numpy(sp).cuda()
    out = torch.full((B, S, topk), -7, dtype=torch.int32, device="cuda")
    C.topk(sh, d_scores, d_sp, out, C.alloc_topk_workspace(sh))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref["topk_idx"])


@pytest.mark.parametrize("kind", ["normal", "coarse", "signed_zero", "spiked16"])
@pytest.mark.parametrize("n_cap,topk", [(8192, 1024), (1000, 100), (4100, 1024), (2049, 2048),
                                        (8192, 700), (3000, 1000)])
def test_topk_many_tokens(kind, n_cap, topk):
    # 2080 tokens: the launch takes the small-block selection (several blocks
    # per CU; rows past 2048 keys try a sampled threshold over a 2048-entry
    # candidate buffer, and fall back to the whole row when it misleads).
    # Causal rows of every length from below K to n_cap, bypass tokens
    # included; 4100 is not a multiple of the per-thread slice.
    B, S = 4, 520
    sh = I.Shape(batch=B, q_per_req=S, ratio=4, n_cap=n_cap, topk=topk, win=8, w_cap=S + 8,
                 heads=1, head_dim=64, rope_dim=0, idx_heads=1, idx_dim=64, out_groups=1,
                 max_len=4 * n_cap, dtype=I.BF16)
    top = 4 * n_cap - S
    sp = np.clip(np.array([top, 4 * topk - 300, 0, 2 * n_cap], np.int64), 0, top).astype(np.int32)
    scores = I.random_scores(n_cap * 7 + topk, B, S, n_cap, kind)
    ref = oracle.run(sh, dict(start_pos=sp), jobs=oracle.JOB_TOPK, scores=scores, nthreads=NTHREADS)
    out = torch.full((B, S, topk), -7, dtype=torch.int32, device="cuda")
    C.topk(sh, torch.from_numpy(scores).cuda(), torch.from_numpy(sp).cuda(), out,
           C.alloc_topk_workspace(sh))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref["topk_idx"])


RANDOM_KINDS = ["normal", "coarse", "signed_zero", "spiked16", "sorted", "rsorted", "clustered", "equal"]


def _random_topk_launch(g, prefill):
    if prefill:   # 2048 tokens or more: the small-block selection of prefill chunks
        B, S = int(g.integers(1, 3)), int(g.integers(2048, 2600))
        n_cap = int(g.choice([2049, 3000, 4096, 6001, 8192]))
        topk = int(g.choice([64, 256, 512, 1000, 1024]))
    else:         # decode launches, rows up to past the two-pass length
        B, S = int(g.integers(1, 7)), int(g.integers(1, 4))
        n_cap = int(g.choice([1024, 4097, 8192, 8193, 9000, 12345, 16384, 20000, 32768, 40000]))
        topk = int(g.choice([1, 7, 64, 256, 257, 512, 1000, 1024, 2048, 4096]))
    max_len = 4 * n_cap + int(g.integers(0, 4))
    sh = I.Shape(batch=B, q_per_req=S, ratio=4, n_cap=n_cap, topk=topk, win=8, w_cap=S + 8, heads=1,
                 head_dim=64, rope_dim=0, idx_heads=1, idx_dim=64, out_groups=1, max_len=max_len,
                 dtype=I.BF16)
    lo = max(0, max_len - S - int(g.integers(1, max_len // 2 + 2)))   # mostly long visible rows
    sp = g.integers(lo, max_len - S + 1, size=B).astype(np.int32)
    kind = RANDOM_KINDS[int(g.integers(0, len(RANDOM_KINDS)))]
    scores = I.random_scores(int(g.integers(0, 1 << 30)), B, S, n_cap, kind)
    ref = oracle.run(sh, dict(start_pos=sp), jobs=oracle.JOB_TOPK, scores=scores, nthreads=NTHREADS)
    out = torch.full((B, S, topk), -7, dtype=torch.int32, device="cuda")
    C.topk(sh, torch.from_numpy(scores).cuda(), torch.from_numpy(sp).cuda(), out, C.alloc_topk_workspace(sh))
    torch.cuda.synchronize()
    return (B, S, n_cap, topk, kind), out.cpu().numpy(), ref["topk_idx"]


@pytest.mark.parametrize("seed", range(40))
def test_topk_random_launches(seed):
    # Seeded random decode launches: batch, tokens, row capacity (every
    # selection form: bypass, whole row, sampled threshold and its fallback,
    # two passes), K from 1 to 4096, positions mostly near the end of the
    # cache, and row kinds from plain to adversarial (monotone rows, a band of
    # winners, one value everywhere).  Four launches per seed; the lists must
    # equal the oracle's bit for bit.
    g = np.random.default_rng([seed, 77])
    for case in range(4):
        what, got, ref = _random_topk_launch(g, prefill=False)
        assert np.array_equal(got, ref), (seed, case, what)


@pytest.mark.parametrize("seed", range(4))
def test_topk_random_prefill_launches(seed):
    # The same for launches of 2048 to 5200 tokens (small blocks, several per CU).
    g = np.random.default_rng([seed, 78])
    what, got, ref = _random_topk_launch(g, prefill=True)
    assert np.array_equal(got, ref), (seed, what)


@pytest.mark.parametrize("topk", [256, 257, 1024])
def test_topk_winners_past_256(topk):
    n_cap = 8192
    sh = I.Shape(batch=1, q_per_req=1, ratio=4, n_cap=n_cap, topk=topk, win=8, w_cap=16, heads=1,
                 head_dim=64, rope_dim=0, idx_heads=1, idx_dim=64, out_groups=1,
                 max_len=4 * n_cap, dtype=I.BF16)
    g = np.random.default_rng(topk)
    scores = g.standard_normal((1, 1, n_cap)).astype(np.float32)
    planted = g.choice(np.arange(257, n_cap), size=200, replace=False)
    scores[0, 0, planted] = 40.0 + g.random(200).astype(np.float32)
    sp = np.array([4 * n_cap - 1], np.int32)
    ref = oracle.run(sh, dict(start_pos=sp), jobs=oracle.JOB_TOPK, scores=scores)
    out = torch.empty((1, 1, topk), dtype=torch.int32, device="cuda")
    C.topk(sh, torch.from_numpy(scores).cuda(), torch.from_numpy(sp).cuda(), out,
           C.alloc_topk_workspace(sh))
    got = out.cpu().numpy()
    assert set(planted.tolist()) <= set(got[0, 0].tolist())
    assert np.array_equal(got, ref["topk_idx"])


# --------------------------------------------------------------------------
# end to end: score -> Top-K -> attention
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cid", [0, 1, 3, 4])
def test_end_to_end(cid, config_inputs):
    cfg = I.CONFIGS[cid]
    sh, inp = cfg.shape, config_inputs(cid)
    ref = oracle_step(sh, inp)
    got = gpu_step(sh, inp)
    rows = U.token_rows(sh, inp["start_pos"])
    bound = U.score_error_bound(sh, inp, rows)
    exempt = U.topk_exemptions(sh, got["topk_idx"], ref["topk_idx"], ref["scores"], bound,
                               inp["start_pos"])
    cap = max(1, sh.batch * sh.q_per_req // 32)
    U.record(f"end_to_end[{cid}]", scored_tokens=len(rows), exemptions=len(exempt), cap=cap,
             exempt=exempt)
    print(f"config {cid}: {len(exempt)} boundary exemptions {exempt}")
    assert len(exempt) <= cap, f"{len(exempt)} boundary exemptions (cap {cap}): {exempt}"
    if "tie:" in cfg.structure:
        # the planted boundary tie (token (0, 0)): its list must be the oracle's
        assert np.array_equal(got["topk_idx"][0, 0], ref["topk_idx"][0, 0]), \
            "token (0, 0) breaks the planted boundary tie differently from the oracle"
    ex = {b * sh.q_per_req + s for (b, s, _) in exempt}
    keep = [t for t in range(sh.batch * sh.q_per_req) if t not in ex]
    U.compare_outputs(sh, got["out"], ref["out"], tokens=keep)


def test_prefill_chunk_full_size():
    # The benchmarked prefill chunk at full size and in the launch
    # configuration the benchmark times (GEMM-shaped score kernel, Top-K in
    # 4-wave blocks): 2 requests x 4096 query tokens, 8 indexer heads,
    # 7168..8192 visible rows per token, K = 1024.  The oracle scores and
    # selects 48 tokens at each end of each request; every other token's list
    # is checked against the exact selection of the scores it was chosen from.
    cfg = I.CONFIGS[5]
    sh, inp = cfg.shape, I.make_inputs(5)
    B, S, K, N = sh.batch, sh.q_per_req, sh.topk, sh.n_cap
    got = gpu_step(sh, inp, jobs=("score", "topk"))
    ends = [(b, s) for b in range(B) for s in list(range(48)) + list(range(S - 48, S))]
    ref_scores = np.full((B, S, N), np.nan, np.float32)
    ref_idx = np.full((B, S, K), -7, np.int32)
    for b in range(B):
        for lo, hi in ((0, 48), (S - 48, S)):
            r = oracle_step(sh, inp, jobs=oracle.JOB_SCORE | oracle.JOB_TOPK,
                            tokens=(b * S + lo, b * S + hi))
            ref_scores[b, lo:hi] = r["scores"][b, lo:hi]
            ref_idx[b, lo:hi] = r["topk_idx"][b, lo:hi]
    rows = [(b, s, n) for (b, s, n) in U.token_rows(sh, inp["start_pos"]) if (b, s) in set(ends)]
    assert len(rows) == len(ends)
    bound = U.score_error_bound(sh, inp, rows)
    for (b, s, n) in rows:
        err = np.abs(got["scores"][b, s, :n].astype(np.float64) - ref_scores[b, s, :n])
        assert np.all(err <= bound[(b, s)]), f"token {(b, s)}: score error above bound"
        assert np.isnan(got["scores"][b, s, n:]).all(), f"token {(b, s)}: invisible rows written"
    exempt = U.topk_exemptions(sh, got["topk_idx"], ref_idx, ref_scores, bound, inp["start_pos"],
                               tokens=ends)
    cap = max(1, len(ends) // 32)
    U.record("prefill_chunk_full_size", checked_tokens=len(ends), exemptions=len(exempt), cap=cap,
             exempt=exempt)
    print(f"prefill chunk: {len(ends)} oracle tokens, {len(exempt)} boundary exemptions {exempt}")
    assert len(exempt) <= cap, f"{len(exempt)} boundary exemptions (cap {cap}): {exempt}"
    # the selection alone, on the oracle's scores, is bit-exact for those tokens
    sc2 = got["scores"].copy()
    for (b, s) in ends:
        sc2[b, s] = ref_scores[b, s]
    got2 = gpu_step(sh, inp, scores=sc2, jobs=("topk",))
    for (b, s) in ends:
        assert np.array_equal(got2["topk_idx"][b, s], ref_idx[b, s]), f"token {(b, s)}"
    # every token: its list is the exact selection of the GPU scores it came from
    nv = np.array([[min((int(inp["start_pos"][b]) + s + 1) // sh.ratio, N) for s in range(S)]
                   for b in range(B)]).reshape(-1)
    want = U.selection_mask(got["scores"].reshape(B * S, N), nv, K)
    have = U.list_mask(got["topk_idx"].reshape(B * S, K), N)
    bad = np.flatnonzero((want != have).any(axis=1))
    assert bad.size == 0, f"{bad.size} tokens whose list is not the selection of their scores: {bad[:8]}"
    gi = got["topk_idx"].reshape(B * S, K)
    assert (np.diff(gi, axis=1) > 0).all(), "lists not ascending"


@pytest.mark.parametrize("n_cap,topk,S,Hi", [(3000, 256, 2, 8), (12000, 1024, 2, 8), (9000, 512, 1, 4)])
def test_end_to_end_exact_grid(n_cap, topk, S, Hi):
    # On the dyadic grid every score is exact on both sides, so GPU scoring
    # plus GPU Top-K must give the oracle's lists with no exemption at all,
    # although the grid makes ties plentiful (lower index wins).
    cfg = small_cfg(q_per_req=S, idx_heads=Hi, n_cap=n_cap, topk=topk, max_len=4 * n_cap,
                    win=64, w_cap=64 + S)
    inp = I.make_inputs(cfg, start_pos=np.array([4 * n_cap - S, 4 * n_cap - 2 * S - 77,
                                                 4 * topk - 1, 4 * topk + 3], np.int32))
    g = np.random.default_rng(n_cap + topk)
    inp["q_idx"] = I.f32_to_bf16_bits((g.integers(-8, 9, inp["q_idx"].shape) / 4.0).astype(np.float32))
    kg = I.f32_to_bf16_bits((g.integers(-8, 9, inp["k_idx"].shape) / 4.0).astype(np.float32))
    inp["k_idx"] = np.where(inp["k_idx"] == I.f32_to_bf16_bits(np.float32([I.POISON]))[0],
                            inp["k_idx"], kg)
    inp["w"] = (g.integers(0, 17, inp["w"].shape) / 16.0).astype(np.float32)
    sh = cfg.shape
    ref = oracle_step(sh, inp)
    got = gpu_step(sh, inp)
    assert np.array_equal(got["scores"], ref["scores"], equal_nan=True)
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])
    U.compare_outputs(sh, got["out"], ref["out"])


def random_grid_case(seed, prefill=False):
    """A seeded random shape inside the supported ranges, with dyadic-grid
    indexer inputs (every score exact on both sides) and, for some seeds,
    an FP8 indexer key cache or every cache paged.  prefill: hundreds of
    tokens per request with 4, 8 or 16 indexer heads, the shape of the
    GEMM-shaped score kernel."""
    g = np.random.default_rng([seed, 77, int(prefill)])
    dt = I.F32 if (g.random() < 0.25 and not prefill) else I.BF16
    ratio = int(g.choice([1, 2, 4, 8])) if not prefill else 4
    B = int(g.integers(1, 7)) if not prefill else int(g.integers(1, 3))
    S = int(g.integers(1, 7)) if not prefill else int(g.integers(128, 701))
    K = int(g.choice([1, 7, 64, 200, 256, 257, 513, 1024]))
    n_cap = int(g.integers(16, 3001)) if not prefill else int(g.integers(S // 4 + 1, 3001))
    max_len = int(g.integers(S, n_cap * ratio + 1))
    win = int(g.integers(1, 301))
    heads = int(g.integers(1, 17))
    divs = [d for d in range(1, heads + 1) if heads % d == 0]
    D = int(g.choice([64, 128]))
    Hi = (int(g.choice([1, 2, 3, 4, 5, 8, 16, 33, 64])) if not prefill
          else int(g.choice([4, 8, 16])))
    cfg = small_cfg(name="random", seed=seed, batch=B, q_per_req=S, ratio=ratio, n_cap=n_cap,
                    topk=K, win=win, w_cap=win + S - 1 + int(g.integers(0, 50)), heads=heads,
                    head_dim=D, rope_dim=int(g.choice([0, 2, 32, D])), idx_heads=Hi,
                    idx_dim=int(g.choice([64, 128])), out_groups=int(g.choice(divs)),
                    max_len=max_len, dtype=dt)
    sh = cfg.shape
    sp = g.integers(0, max_len - S + 1, size=B).astype(np.int32)
    inp = I.make_inputs(cfg, start_pos=sp)
    def grid(shape):
        v = (g.integers(-8, 9, shape) / 4.0).astype(np.float32)
        return I.f32_to_bf16_bits(v) if dt == I.BF16 else v
    inp["q_idx"] = grid(inp["q_idx"].shape)
    poison = (I.f32_to_bf16_bits(np.float32([I.POISON]))[0] if dt == I.BF16
              else np.float32(I.POISON))
    inp["k_idx"] = np.where(inp["k_idx"] == poison, inp["k_idx"], grid(inp["k_idx"].shape))
    inp["w"] = (g.integers(0, 17, inp["w"].shape) / 16.0).astype(np.float32)
    if dt == I.BF16 and g.random() < (0.5 if prefill else 0.3):
        # FP8 key cache: every grid value m/4 (|m| <= 8) is an E4M3 value, so
        # codes hold the same keys (poisoned rows: the largest finite code,
        # 448); prefill cases scale each row by a random power of two, which
        # keeps every score exact
        kf = I.bf16_bits_to_f32(inp["k_idx"])
        codes = I.f32_to_e4m3_bits(np.where(kf == np.float32(I.POISON), np.float32(448.0), kf))
        inp["k_idx8"] = codes
        inp["k_scale"] = (np.exp2(g.integers(-2, 3, size=inp["k_idx"].shape[:2])).astype(np.float32)
                          if prefill else np.ones(inp["k_idx"].shape[:2], dtype=np.float32))
        del inp["k_idx"]
    if g.random() < 0.3:
        inp = I.page_inputs(inp, int(g.choice([16, 32, 64])), seed=seed, win=True)
    return sh, inp


@pytest.mark.parametrize("seed,prefill", [(k, False) for k in range(64)] + [(k, True) for k in range(18)])
def test_random_shapes_exact_grid(seed, prefill):
    # scores and lists bitwise, attention within tolerance, over random
    # shapes: ratio, batch, tokens per request, K (bypass and not), capacities,
    # head and group counts, RoPE dims, fp32 and bf16, dense and paged caches;
    # prefill-shaped cases reach the GEMM-shaped score kernel
    sh, inp = random_grid_case(seed, prefill)
    paged = "cmp_table" in inp
    print(f"seed {seed}: {sh} paged={paged}", flush=True)
    ref = oracle.run_paged(sh, inp, nthreads=NTHREADS) if paged else oracle_step(sh, inp)
    got = gpu_step(sh, inp)
    assert np.array_equal(got["scores"], ref["scores"], equal_nan=True)
    assert np.array_equal(got["topk_idx"], ref["topk_idx"])
    U.compare_outputs(sh, got["out"], ref["out"])


def random_long_rows_case(seed):
    """A seeded random decode shape whose rows run past 8192 keys (the
    one-workgroup Top-K's sampled-threshold path), N(0,1) inputs."""
    g = np.random.default_rng([seed, 991])
    B, S = int(g.integers(1, 4)), int(g.integers(1, 4))
    K = int(g.choice([64, 256, 257, 512, 1024, 2048]))
    n_cap = int(g.integers(8193, 40001))
    max_len = int(g.integers(4 * 8000, n_cap * 4 + 1))
    win, heads = int(g.integers(1, 257)), int(g.integers(1, 17))
    divs = [d for d in range(1, heads + 1) if heads % d == 0]
    D = int(g.choice([64, 128]))
    cfg = small_cfg(name="long", seed=seed, batch=B, q_per_req=S, ratio=4, n_cap=n_cap, topk=K, win=win,
                    w_cap=win + S - 1 + int(g.integers(0, 50)), heads=heads, head_dim=D,
                    rope_dim=int(g.choice([0, 32, D])), idx_heads=int(g.choice([1, 4, 8, 16])),
                    idx_dim=int(g.choice([64, 128])), out_groups=int(g.choice(divs)), max_len=max_len,
                    dtype=I.BF16)
    sp = g.integers(max_len // 2, max_len - S + 1, size=B).astype(np.int32)
    return cfg.shape, I.make_inputs(cfg, start_pos=sp, structure="none")


@pytest.mark.parametrize("seed", range(24))
def test_random_long_rows(seed):
    # rows of 8k-40k keys and K from 64 to 2048: scores within the bound,
    # unscored entries untouched, and the Top-K lists bitwise on the
    # oracle's own scores
    sh, inp = random_long_rows_case(seed)
    print(f"seed {seed}: {sh}", flush=True)
    ref = oracle_step(sh, inp, jobs=oracle.JOB_SCORE | oracle.JOB_TOPK)
    got = gpu_step(sh, inp, jobs=("score",))
    check_scores(sh, inp, got, ref)
    lists = gpu_step(sh, inp, scores=ref["scores"], jobs=("topk",))["topk_idx"]
    assert np.array_equal(lists, ref["topk_idx"])


def test_determinism(config_inputs):
    cid = 3
    sh, inp = I.CONFIGS[cid].shape, config_inputs(cid)
    a = gpu_step(sh, inp)
    b = gpu_step(sh, inp)
    for k in ("scores", "topk_idx", "out"):
        assert np.array_equal(a[k], b[k], equal_nan=True), k


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------

EDGE = {
    # early positions: empty compressed stream, partial windows, bypass
    "early": dict(batch=6, q_per_req=1, topk=64, win=64, w_cap=64, start=[0, 1, 2, 3, 63, 64]),
    # n_vis == K and K + 1 in one batch (bypass boundary), S = 3 causal tokens
    "bypass_edge": dict(batch=4, q_per_req=3, topk=64, win=32, w_cap=40,
                        start=[4 * 64 - 3, 4 * 64 - 2, 4 * 65 - 3, 900]),
    # ring wrap with spare capacity, two groups, 8 heads
    "ring_groups": dict(batch=3, q_per_req=4, win=48, w_cap=53, heads=8, out_groups=2,
                        start=[5, 700, 1019]),
    # head_dim 64 bf16, no RoPE, four groups
    "d64_norope": dict(batch=3, q_per_req=2, head_dim=64, rope_dim=0, heads=12, out_groups=4,
                       idx_dim=64, start=[10, 400, 1000]),
    # fp32, head_dim 128, one head
    "f32_one_head": dict(batch=2, q_per_req=2, dtype=I.F32, heads=1, rope_dim=16,
                         start=[300, 1021]),
    # wide Top-K relative to the window, many splits
    "many_splits": dict(batch=2, q_per_req=1, topk=600, win=300, w_cap=300, n_cap=1024,
                        max_len=4096, start=[4095, 3000]),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases(name):
    kw = dict(EDGE[name])
    start = np.array(kw.pop("start"), np.int32)
    cfg = small_cfg(name=name, **kw)
    sh = cfg.shape
    inp = I.make_inputs(cfg, start_pos=start)
    ref = oracle_step(sh, inp)
    got = gpu_step(sh, inp)
    rows = U.token_rows(sh, inp["start_pos"])
    bound = U.score_error_bound(sh, inp, rows)
    exempt = U.topk_exemptions(sh, got["topk_idx"], ref["topk_idx"], ref["scores"], bound,
                               inp["start_pos"])
    assert not exempt
    U.compare_outputs(sh, got["out"], ref["out"])
    # attention alone on the oracle's lists
    got2 = gpu_step(sh, inp, topk_idx=ref["topk_idx"], jobs=("attn",))
    U.compare_outputs(sh, got2["out"], ref["out"])


def test_padding_and_out_of_range_indices():
    cfg = small_cfg(batch=2, q_per_req=1)
    sh = cfg.shape
    inp = I.make_inputs(cfg, start_pos=np.array([800, 1000], np.int32))
    ti = oracle_step(sh, inp)["topk_idx"]
    bad = ti.copy()
    bad[0, 0, :5] = [-1, sh.n_cap, sh.n_cap + 100, -100, 2 ** 30]
    ref = oracle_step(sh, inp, jobs=oracle.JOB_ATTN, topk_idx=bad)
    got = gpu_step(sh, inp, topk_idx=bad, jobs=("attn",))
    U.compare_outputs(sh, got["out"], ref["out"])


def test_empty_batch_is_a_noop():
    sh = small_cfg().shape.replace(batch=0)
    z = torch.zeros(16, dtype=torch.int32, device="cuda")
    f = torch.zeros(16, dtype=torch.float32, device="cuda")
    h = torch.zeros(16, dtype=torch.bfloat16, device="cuda")   # the shape's dtype is bf16
    r = torch.zeros((1, sh.rope_dim // 2), dtype=torch.float32, device="cuda")  # one table row
    C.indexer_score(sh, h, f, h, z, f)
    C.topk(sh, f, z, z)
    C.sparse_attn_decode(sh, h, h, h, h, h, z, z, r, r, 0.1, h, f)
    torch.cuda.synchronize()
    assert int(z.abs().sum()) == 0 and float(f.abs().sum()) == 0.0 and float(h.float().abs().sum()) == 0.0


def test_binding_refuses_short_or_mistyped_tensors():
    # the C ABI takes pointers only: the binding checks every tensor against
    # the shape before any launch, so nothing runs past a buffer's end
    cfg = small_cfg()
    sh, inp = cfg.shape, I.make_inputs(cfg)
    d = C.to_device(inp, sh)
    bufs = C.alloc_outputs(sh)
    with pytest.raises(ValueError, match="k_idx"):
        C.indexer_score(sh, d["q_idx"], d["w"], d["k_idx"][:-1], d["start_pos"], bufs["scores"])
    with pytest.raises(TypeError, match="w"):
        C.indexer_score(sh, d["q_idx"], d["w"].double(), d["k_idx"], d["start_pos"], bufs["scores"])
    with pytest.raises(ValueError, match="topk_idx"):
        C.topk(sh, bufs["scores"], d["start_pos"], bufs["topk_idx"].reshape(-1)[:-1])
    with pytest.raises(ValueError, match="v_cmp"):
        C.sparse_attn_decode(sh, d["q"], d["k_win"], d["v_win"], d["k_cmp"], d["v_cmp"][:1],
                             bufs["topk_idx"], d["start_pos"], d["rope_cos"], d["rope_sin"],
                             I.softmax_scale(sh), bufs["out"], bufs["attn_ws"])
    with pytest.raises(ValueError, match="rope_sin"):
        C.sparse_attn_decode(sh, d["q"], d["k_win"], d["v_win"], d["k_cmp"], d["v_cmp"],
                             bufs["topk_idx"], d["start_pos"], d["rope_cos"], d["rope_sin"][:, :1].contiguous(),
                             I.softmax_scale(sh), bufs["out"], bufs["attn_ws"])
    torch.cuda.synchronize()


def test_refused_call_leaves_outputs_untouched():
    # K = 1024 rows do not fit one workgroup per token: the split kernels and
    # their workspace
    cfg = small_cfg(batch=2, q_per_req=1, topk=1024)
    sh = cfg.shape
    assert C.sparse_attn_workspace_bytes(sh) > 16
    inp = I.make_inputs(cfg)
    d = C.to_device(inp, sh)
    bufs = C.alloc_outputs(sh)
    bufs["out"].fill_(3.0)
    small_ws = bufs["attn_ws"][:16]
    with pytest.raises(C.CsaError) as e:
        C.sparse_attn_decode(sh, d["q"], d["k_win"], d["v_win"], d["k_cmp"], d["v_cmp"],
                             bufs["topk_idx"], d["start_pos"], d["rope_cos"], d["rope_sin"], 0.1,
                             bufs["out"], small_ws)
    assert e.value.code == 6
    torch.cuda.synchronize()
    assert bool((bufs["out"] == 3.0).all())
