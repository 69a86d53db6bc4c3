"""Seeded synthetic inputs for the CSA sparse-attention decode step.

This module only draws and lays out data: it holds none of the step's own
arithmetic (no scoring, selection, softmax or rotation of outputs).  The CPU
oracle and the HIP path both consume what it returns, so the two always see
bit-identical inputs.

Every tensor comes from its own child stream ``np.random.default_rng([seed,
tensor_id])`` in a fixed tensor order, so one tensor can be regenerated
without drawing the others.  Floating-point values are drawn in float32 and,
for the bf16 configurations, rounded to bf16 with round-to-nearest-even;
bf16 tensors are returned as ``np.uint16`` bit patterns.

Workload shapes follow the pages' decode setting ("Perf: skip redundant CSA
scoring and fuse gather unpack", description: ratio-4 compressed cache, Top-K
with a bypass when the cache fits; "Perf: fuse HCA merge, inverse RoPE, and
packing", description: B=16, S=8, 64 compressed rows, two output groups).
No public dataset is involved: all structure (lengths, planted winners,
duplicated rows, poison) is synthetic and documented per configuration.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
from typing import Dict, Optional

import numpy as np

# Value written into every cache row the step must not read (compressed rows
# past the causal horizon, ring slots outside the live window).  A leak of such
# a row into a score or a softmax changes the result by orders of magnitude.
POISON = 1.0e4

F32 = 0
BF16 = 1

# tensor ids of the child streams (fixed order; never renumber)
_T_START, _T_Q, _T_KWIN, _T_VWIN, _T_KCMP, _T_VCMP, _T_QIDX, _T_W, _T_KIDX, _T_STRUCT, _T_TIE = range(11)


@dataclasses.dataclass(frozen=True)
class Shape:
    """Problem sizes of one decode step (field names match the C ABI)."""

    batch: int          # B requests
    q_per_req: int      # S query tokens per request (positions start_pos+0 .. start_pos+S-1)
    ratio: int          # R raw tokens per compressed row
    n_cap: int          # compressed rows allocated per request
    topk: int           # K (IDX_TOPK)
    win: int            # sliding-window length
    w_cap: int          # ring capacity of the window cache
    heads: int          # H query heads (one shared KV head)
    head_dim: int       # D
    rope_dim: int       # Dr: the last Dr dims carry interleaved RoPE pairs
    idx_heads: int      # Hi indexer heads
    idx_dim: int        # Di indexer head dim
    out_groups: int     # G output head groups
    max_len: int        # host bound: max_b start_pos[b] + S
    dtype: int          # F32 or BF16

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    shape: Shape
    seed: int
    lengths: str          # how start_pos is drawn (documentation + dispatch key)
    structure: str        # extra structure planted into the indexer keys ("+"-separated parts)
    supplied_topk: bool   # True: the harness supplies topk_idx (attention only)
    indexer_only: bool = False  # True: a prefill chunk measured for scoring + Top-K


def _shape(**kw) -> Shape:
    return Shape(**kw)


CONFIGS: Dict[int, Config] = {
    0: Config(
        name="tiny_fp32",
        shape=_shape(batch=1, q_per_req=1, ratio=4, n_cap=256, topk=64, win=64, w_cap=64,
                     heads=4, head_dim=64, rope_dim=32, idx_heads=2, idx_dim=64,
                     out_groups=1, max_len=1024, dtype=F32),
        seed=0, lengths="fixed:1024", structure="none", supplied_topk=False),
    1: Config(
        name="bypass",
        shape=_shape(batch=16, q_per_req=1, ratio=4, n_cap=256, topk=512, win=128, w_cap=128,
                     heads=16, head_dim=128, rope_dim=64, idx_heads=4, idx_dim=128,
                     out_groups=1, max_len=1024, dtype=BF16),
        seed=1, lengths="start_uniform:0:1023", structure="none", supplied_topk=False),
    2: Config(
        name="hca_merge",
        shape=_shape(batch=16, q_per_req=8, ratio=4, n_cap=64, topk=64, win=128, w_cap=256,
                     heads=16, head_dim=128, rope_dim=64, idx_heads=4, idx_dim=128,
                     out_groups=2, max_len=4096 + 8, dtype=BF16),
        seed=2, lengths="start_uniform:0:4095", structure="none", supplied_topk=True),
    3: Config(
        name="long_context",
        shape=_shape(batch=16, q_per_req=1, ratio=4, n_cap=16384, topk=512, win=128, w_cap=128,
                     heads=16, head_dim=128, rope_dim=64, idx_heads=4, idx_dim=128,
                     out_groups=1, max_len=65536, dtype=BF16),
        seed=3, lengths="len_uniform:32768:65536", structure="planted:256", supplied_topk=False),
    4: Config(
        name="wide_topk",
        shape=_shape(batch=64, q_per_req=2, ratio=4, n_cap=32768, topk=1024, win=256, w_cap=512,
                     heads=16, head_dim=128, rope_dim=64, idx_heads=8, idx_dim=128,
                     out_groups=1, max_len=131072, dtype=BF16),
        # 1% duplicated key rows, and the row that token (0, 0) ranks K-th (row
        # 13692, found by the oracle on the inputs without the tie:
        # tests/golden/config4_boundary_tie.py) copied to 2 rows below and 2
        # above it, so that equal scores straddle the selection boundary
        seed=4, lengths="fixed:131072", structure="dup:0.01+tie:0:13692:2:2", supplied_topk=False),
    # A prefill chunk: the last 4096 tokens of a 32768-token context, each
    # scoring its own causally visible compressed rows (7168 .. 8192).
    5: Config(
        name="prefill_chunk",
        shape=_shape(batch=2, q_per_req=4096, ratio=4, n_cap=8192, topk=1024, win=128, w_cap=4224,
                     heads=16, head_dim=128, rope_dim=64, idx_heads=8, idx_dim=128,
                     out_groups=1, max_len=32768, dtype=BF16),
        seed=5, lengths="fixed:32768", structure="none", supplied_topk=False, indexer_only=True),
}


# ----------------------------------------------------------------------------
# dtype helpers (data formatting only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return uint16 bits.

    For finite inputs the biased sum stays below 2**32, so uint32 arithmetic
    cannot wrap.
    """
    u = np.array(x, dtype=np.float32, copy=True, order="C").view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


E4M3_MAX = 448.0


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Encode values as OCP FP8 E4M3 codes (uint8): round to nearest, ties to
    even; magnitudes past the largest finite value (448) saturate to it.

    Data formatting of the FP8 indexer key cache the inputs carry; the kernels
    and the oracle only decode.  NaN inputs are not expected.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # binade exponent of a, floored at the smallest normal binade (2^-6)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))   # a = m * 2^ex, m in [0.5, 1)
    e = np.clip(ex - 1, -6, 8)
    q = np.rint(a / np.exp2(e - 3))              # 3 fraction bits: q in [0, 16]
    up = q >= 16                                 # rounded into the next binade
    e = np.where(up, e + 1, e)
    q = np.where(up, 8, q)
    over = (e > 8) | ((e == 8) & (q > 14))       # past 1.75 * 2^8: saturate
    e = np.where(over, 8, e)
    q = np.where(over, 14, q)
    normal = q >= 8                              # else a subnormal (e == -6)
    field = np.where(normal, e + 7, 0).astype(np.uint8)
    man = np.where(normal, q - 8, q).astype(np.uint8)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    return (sign | (field << np.uint8(3)) | man).astype(np.uint8)


def quantize_rows_e4m3(k: np.ndarray):
    """Per-row FP8 E4M3 quantisation of float32 rows [..., Di]: scale = amax / 448
    (1 for an all-zero row), codes = E4M3(k / scale).  Returns (codes uint8,
    scales float32)."""
    k = np.asarray(k, dtype=np.float32)
    amax = np.abs(k).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    codes = f32_to_e4m3_bits(k / scale[..., None])
    return codes, scale


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_float(a: np.ndarray, dtype: int) -> np.ndarray:
    """Values of an input tensor as float32 (exact for both storage types)."""
    return bf16_bits_to_f32(a) if dtype == BF16 else np.asarray(a, dtype=np.float32)


def _store(x: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid])


def _normal(seed: int, tid: int, shape) -> np.ndarray:
    return _rng(seed, tid).standard_normal(size=shape, dtype=np.float32)


# ----------------------------------------------------------------------------
# positions, RoPE tables
# ----------------------------------------------------------------------------

def draw_start_pos(cfg: Config, seed: int, shape: Shape) -> np.ndarray:
    """start_pos[b]: position of request b's first query token."""
    kind, *args = cfg.lengths.split(":")
    B, S = shape.batch, shape.q_per_req
    g = _rng(seed, _T_START)
    if kind == "fixed":            # context L for every request: last token at L-1
        L = int(args[0])
        sp = np.full(B, L - S, dtype=np.int64)
    elif kind == "start_uniform":  # start positions uniform on [lo, hi]
        lo, hi = int(args[0]), int(args[1])
        sp = g.integers(lo, hi + 1, size=B)
    elif kind == "len_uniform":    # context lengths uniform on [lo, hi], last token at L-1
        lo, hi = int(args[0]), int(args[1])
        sp = g.integers(lo, hi + 1, size=B) - S
    else:
        raise ValueError(cfg.lengths)
    return np.ascontiguousarray(sp, dtype=np.int32)


def rope_tables(rows: int, rope_dim: int, base: float = 10000.0):
    """cos/sin tables [rows][rope_dim/2] in float32 for interleaved RoPE pairs.

    Pair i (dims 2i, 2i+1 of the RoPE block) turns by angle p * base^(-2i/rope_dim)
    at position p.  Angles and trig are evaluated in float64 and rounded once.
    """
    half = rope_dim // 2
    if half == 0:
        z = np.zeros((rows, 0), dtype=np.float32)
        return z, z.copy()
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / rope_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# ----------------------------------------------------------------------------
# the full input set
# ----------------------------------------------------------------------------

def visible_rows(p: np.ndarray, ratio: int) -> np.ndarray:
    """Compressed rows whose whole raw-token block lies at or before position p.

    Used only to decide which rows to poison; the oracle and the kernels derive
    visibility themselves.
    """
    return (np.asarray(p, dtype=np.int64) + 1) // ratio


def _plant(part: str, g: np.random.Generator, g_tie: np.random.Generator, k_idx: np.ndarray,
           q_idx: np.ndarray, w: np.ndarray, last_vis: np.ndarray, sh: Shape) -> None:
    """Apply one structure part to the float32 indexer keys k_idx [B, N_cap, Di] in place."""
    B, Di, dt = sh.batch, sh.idx_dim, sh.dtype
    kind, _, arg = part.partition(":")
    if kind == "planted":
        # Rows aligned with the request's weighted indexer query score far above
        # the N(0,1) rows, so they must win Top-K wherever they sit.
        n_plant = int(arg)
        qi = as_float(_store(q_idx, dt), dt).astype(np.float64)
        for b in range(B):
            nv = int(last_vis[b])
            if nv <= sh.topk:
                continue
            m = min(n_plant, nv)
            pos = g.choice(nv, size=m, replace=False)
            u = np.einsum("h,hc->c", w[b, 0].astype(np.float64), qi[b, 0])
            u /= np.linalg.norm(u)
            alpha = g.uniform(1.0, 2.0, size=m)
            k_idx[b, pos] = (alpha[:, None] * np.sqrt(Di) * u[None, :]).astype(np.float32)
    elif kind == "dup":
        # A fraction of rows copy another row's indexer key, so exact score ties
        # occur on both sides of every comparison.
        frac = float(arg)
        for b in range(B):
            nv = int(last_vis[b])
            nd = int(round(frac * nv))
            if nd == 0 or nv < 2:
                continue
            dst = g.choice(nv, size=nd, replace=False)
            src = g.integers(0, nv, size=nd)
            k_idx[b, dst] = k_idx[b, src]
    elif kind == "tie":
        # tie:b:row:below:above -- key row `row` of request b is copied to
        # `below` seeded random rows under it and `above` rows over it (among
        # the rows its last token sees), so equal scores sit on both sides of
        # that row's index.  Which row to copy is chosen by the caller: the
        # wide Top-K configuration names the row its first token ranks K-th,
        # so the tie straddles the selection boundary and the index decides.
        b, row, below, above = (int(x) for x in arg.split(":"))
        nv = int(last_vis[b])
        assert 0 <= row < nv and below <= row and above <= nv - 1 - row
        lo = g_tie.choice(row, size=below, replace=False) if below else np.zeros(0, np.int64)
        hi = row + 1 + g_tie.choice(nv - 1 - row, size=above, replace=False) if above else np.zeros(0, np.int64)
        k_idx[b, np.concatenate([lo, hi])] = k_idx[b, row]
    elif kind != "none":
        raise ValueError(part)


def make_inputs(cfg_id_or_cfg, seed: Optional[int] = None, poison: bool = True,
                shape: Optional[Shape] = None, start_pos: Optional[np.ndarray] = None,
                structure: Optional[str] = None, key_format: str = "bf16",
                indexer_only: bool = False) -> Dict[str, np.ndarray]:
    """Draw every input of one decode step.

    Returns a dict of contiguous numpy arrays:
      start_pos [B] int32, q [B,S,H,D], k_win/v_win [B,W_cap,D],
      k_cmp/v_cmp [B,N_cap,D], q_idx [B,S,Hi,Di], w [B,S,Hi] float32,
      k_idx [B,N_cap,Di], rope_cos/rope_sin [max_len, Dr/2] float32 and,
      for configurations whose harness supplies the selection,
      topk_idx [B,S,K] int32.
    Storage is uint16 (bf16 bits) or float32 according to shape.dtype.
    With key_format="fp8" the indexer keys come instead as an FP8 cache:
    k_idx8 [B,N_cap,Di] uint8 E4M3 codes and k_scale [B,N_cap] float32, each
    row quantised from the keys drawn above (so planted rows, duplicated
    rows and poison keep their meaning); k_idx is then left out.
    With indexer_only only start_pos, q_idx, w and the indexer keys are drawn
    (each tensor has its own child stream, so their values do not change).
    """
    cfg = CONFIGS[cfg_id_or_cfg] if isinstance(cfg_id_or_cfg, int) else cfg_id_or_cfg
    sh = shape or cfg.shape
    seed = cfg.seed if seed is None else seed
    structure = cfg.structure if structure is None else structure
    B, S, H, D = sh.batch, sh.q_per_req, sh.heads, sh.head_dim
    Hi, Di, Nc, Wc = sh.idx_heads, sh.idx_dim, sh.n_cap, sh.w_cap
    dt = sh.dtype

    sp = draw_start_pos(cfg, seed, sh) if start_pos is None else np.ascontiguousarray(start_pos, np.int32)
    assert sp.shape == (B,)
    assert int(sp.min(initial=0)) >= 0 and int((sp + S).max(initial=0)) <= sh.max_len

    # Independent child streams: drawing them on threads changes no value.
    jobs = dict(q=(_T_Q, (B, S, H, D)), k_win=(_T_KWIN, (B, Wc, D)), v_win=(_T_VWIN, (B, Wc, D)),
                k_cmp=(_T_KCMP, (B, Nc, D)), v_cmp=(_T_VCMP, (B, Nc, D)),
                q_idx=(_T_QIDX, (B, S, Hi, Di)), k_idx=(_T_KIDX, (B, Nc, Di)))
    if indexer_only:
        jobs = {k: v for k, v in jobs.items() if k in ("q_idx", "k_idx")}
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        futs = {k: ex.submit(_normal, seed, tid, shp) for k, (tid, shp) in jobs.items()}
        drawn = {k: f.result() for k, f in futs.items()}
    q, k_win, v_win = drawn.get("q"), drawn.get("k_win"), drawn.get("v_win")
    k_cmp, v_cmp, q_idx, k_idx = drawn.get("k_cmp"), drawn.get("v_cmp"), drawn["q_idx"], drawn["k_idx"]
    w = _rng(seed, _T_W).random(size=(B, S, Hi), dtype=np.float32)

    g = _rng(seed, _T_STRUCT)
    last_vis = np.minimum(visible_rows(sp + S - 1, sh.ratio), Nc)   # rows visible to the last token
    for part in structure.split("+"):
        _plant(part, g, _rng(seed, _T_TIE), k_idx, q_idx, w, last_vis, sh)

    if poison:
        for b in range(B):
            nv = int(last_vis[b])
            k_idx[b, nv:] = POISON
            if indexer_only:
                continue
            if not cfg.supplied_topk:
                k_cmp[b, nv:] = POISON
                v_cmp[b, nv:] = POISON
            lo = max(0, int(sp[b]) - sh.win + 1)
            hi = int(sp[b]) + S - 1
            live = np.zeros(Wc, dtype=bool)
            live[np.arange(lo, hi + 1) % Wc] = True
            k_win[b, ~live] = POISON
            v_win[b, ~live] = POISON

    raw = dict(q=q, k_win=k_win, v_win=v_win, k_cmp=k_cmp, v_cmp=v_cmp, q_idx=q_idx, k_idx=k_idx)
    raw = {k: v for k, v in raw.items() if v is not None}
    del q, k_win, v_win, k_cmp, v_cmp, q_idx, k_idx, drawn
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(raw)) as ex:
        futs = {k: ex.submit(_store, v, dt) for k, v in raw.items()}
        out = {k: f.result() for k, f in futs.items()}
    del raw
    out.update(start_pos=sp, w=np.ascontiguousarray(w, np.float32))
    if not indexer_only:
        cos, sin = rope_tables(sh.max_len, sh.rope_dim)
        out.update(rope_cos=cos, rope_sin=sin)
    if key_format == "fp8":
        kf = out.pop("k_idx")
        codes = np.empty(kf.shape, dtype=np.uint8)
        scales = np.empty(kf.shape[:2], dtype=np.float32)
        for b in range(B):   # one request at a time keeps the float64 temporaries small
            codes[b], scales[b] = quantize_rows_e4m3(as_float(kf[b], dt))
        out.update(k_idx8=codes, k_scale=scales)
    elif key_format != "bf16":
        raise ValueError(key_format)
    if cfg.supplied_topk and not indexer_only:
        # The HCA-shaped case attends every compressed row it is given.
        K = sh.topk
        ti = np.full((B, S, K), -1, dtype=np.int32)
        n = min(K, Nc)
        ti[:, :, :n] = np.arange(n, dtype=np.int32)
        out["topk_idx"] = ti
    return out


def page_cache(dense: np.ndarray, block_size: int, seed: int, spare_blocks: int = 3,
               fill=None):
    """Lay a dense per-request cache [B, n_cap, ...] out as a pool of blocks.

    Returns (pool [n_blocks, block_size, ...], table [B, ceil(n_cap/block_size)]
    int32): the blocks of all requests in a seeded random order, plus
    `spare_blocks` blocks that no table entry names, filled with `fill` (the
    poison value by default) so that a wrong mapping reads them.  Data layout
    only: logical row j of request b is pool row
    table[b, j // block_size] * block_size + j % block_size.
    """
    B, n_cap = dense.shape[:2]
    bpr = -(-n_cap // block_size)
    pad = bpr * block_size - n_cap
    d = dense
    if pad:
        d = np.concatenate([dense, np.repeat(dense[:, -1:], pad, axis=1)], axis=1)
    blocks = d.reshape(B * bpr, block_size, *dense.shape[2:])
    n_blocks = B * bpr + spare_blocks
    g = np.random.default_rng([seed, 555])
    perm = g.permutation(n_blocks)
    pool = np.empty((n_blocks, block_size) + dense.shape[2:], dtype=dense.dtype)
    if fill is None:
        fill = f32_to_bf16_bits(np.float32([POISON]))[0] if dense.dtype == np.uint16 else POISON
    pool[perm[B * bpr:]] = fill
    pool[perm[:B * bpr]] = blocks
    table = perm[:B * bpr].reshape(B, bpr).astype(np.int32)
    return pool, table


def page_inputs(inp: dict, block_size: int, seed: int, idx: bool = True, cmp: bool = True,
                spare_blocks: int = 3, win: bool = False) -> dict:
    """A copy of a seeded input dict with the indexer key cache (idx), the
    compressed K/V cache (cmp) and/or the window rings (win) moved into block
    pools (page_cache).  Names: k_idx_pool (or k_idx8_pool + k_scale_pool),
    idx_table, idx_block_size; k_cmp_pool + v_cmp_pool sharing cmp_table,
    cmp_block_size; k_win_pool + v_win_pool sharing win_table, win_block_size
    (logical row = ring slot).  The dense arrays that were paged are dropped."""
    out = dict(inp)
    if win:
        out["k_win_pool"], out["win_table"] = page_cache(inp["k_win"], block_size, seed + 2,
                                                         spare_blocks)
        out["v_win_pool"], _ = page_cache(inp["v_win"], block_size, seed + 2, spare_blocks)
        del out["k_win"], out["v_win"]
        out["win_block_size"] = block_size
    if idx:
        if "k_idx8" in inp:
            out["k_idx8_pool"], out["idx_table"] = page_cache(inp["k_idx8"], block_size, seed,
                                                              spare_blocks, fill=0x7E)
            out["k_scale_pool"], _ = page_cache(inp["k_scale"], block_size, seed, spare_blocks)
            del out["k_idx8"], out["k_scale"]
            out.pop("k_idx", None)
        else:
            out["k_idx_pool"], out["idx_table"] = page_cache(inp["k_idx"], block_size, seed,
                                                             spare_blocks)
            del out["k_idx"]
        out["idx_block_size"] = block_size
    if cmp:
        out["k_cmp_pool"], out["cmp_table"] = page_cache(inp["k_cmp"], block_size, seed + 1,
                                                         spare_blocks)
        out["v_cmp_pool"], _ = page_cache(inp["v_cmp"], block_size, seed + 1, spare_blocks)
        del out["k_cmp"], out["v_cmp"]
        out["cmp_block_size"] = block_size
    return out


def paged_ring_slot_mapping(shape: Shape, start_pos: np.ndarray, win_table: np.ndarray,
                            block_size: int) -> np.ndarray:
    """Slot mapping of the step's new tokens into paged window rings: token
    (b, s) at position p = start_pos[b] + s belongs in ring slot r = p mod w_cap,
    which is pool row win_table[b, r // block_size] * block_size + r % block_size
    of the pool viewed as one flat cache.  Shape [B*S] int32."""
    B, S = shape.batch, shape.q_per_req
    p = np.asarray(start_pos, dtype=np.int64)[:, None] + np.arange(S)[None, :]
    r = p % shape.w_cap
    tab = np.asarray(win_table, dtype=np.int64)
    rows = tab[np.arange(B)[:, None], r // block_size] * block_size + r % block_size
    return rows.reshape(-1).astype(np.int32)


def ring_slot_mapping(shape: Shape, start_pos: np.ndarray) -> np.ndarray:
    """Slot mapping of the step's new tokens into the per-request window rings
    viewed as one flat cache [B*w_cap][D]: token (b, s) at position
    p = start_pos[b] + s goes to row b*w_cap + p mod w_cap.  Shape [B*S] int32."""
    B, S, Wc = shape.batch, shape.q_per_req, shape.w_cap
    p = np.asarray(start_pos, np.int64)[:, None] + np.arange(S)[None, :]
    return (np.arange(B)[:, None] * Wc + p % Wc).reshape(-1).astype(np.int32)


def softmax_scale(shape: Shape) -> float:
    """fp32(1/sqrt(D)), the scale every configuration uses."""
    return float(np.float32(1.0 / np.sqrt(shape.head_dim)))


def random_scores(seed: int, B: int, S: int, n_cap: int, kind: str = "normal") -> np.ndarray:
    """Synthetic fp32 score rows for exercising selection on its own."""
    g = np.random.default_rng([seed, 101])
    if kind == "normal":
        return g.standard_normal(size=(B, S, n_cap), dtype=np.float32)
    if kind == "coarse":   # few distinct values: heavy ties
        return (g.integers(-8, 9, size=(B, S, n_cap)) / 4.0).astype(np.float32)
    if kind.startswith("spiked"):
        # large values exactly at row positions i with (i // 1024) == (i % 1024) % m:
        # a strided sample of the row then sees only the spikes
        m = int(kind[len("spiked"):])
        v = g.standard_normal(size=(B, S, n_cap), dtype=np.float32)
        i = np.arange(n_cap)
        v[..., (i // 1024) == (i % 1024) % m] += 100.0
        return v
    if kind == "signed_zero":
        s = g.integers(0, 3, size=(B, S, n_cap)).astype(np.float32) - 1.0
        z = g.random(size=(B, S, n_cap)) < 0.5
        s[(s == 0) & z] = -0.0
        return s
    if kind in ("sorted", "rsorted"):   # monotone rows: the winners sit at one end
        v = np.sort(g.standard_normal(size=(B, S, n_cap), dtype=np.float32), axis=-1)
        return v if kind == "sorted" else np.ascontiguousarray(v[..., ::-1])
    if kind == "clustered":   # a band of 3000 high scores at a random offset in each row
        v = g.standard_normal(size=(B, S, n_cap), dtype=np.float32)
        for r in v.reshape(-1, n_cap):
            a = int(g.integers(0, n_cap))
            r[a:a + 3000] += 6.0
        return v
    if kind == "equal":   # one value everywhere: only the row index decides
        return np.full((B, S, n_cap), 1.5, np.float32)
    raise ValueError(kind)
