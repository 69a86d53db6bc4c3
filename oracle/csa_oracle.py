"""ctypes wrapper of oracle.c (test infrastructure; see oracle.c's header).

The wrapper marshals numpy arrays only; every step of the computation is in
oracle.c.  It does not import the product package: any object with the shape
fields (batch, q_per_req, ratio, ...) is accepted.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

JOB_SCORE, JOB_TOPK, JOB_ATTN = 1, 2, 4

_FIELDS = ("batch", "q_per_req", "ratio", "n_cap", "topk", "win", "w_cap", "heads",
           "head_dim", "rope_dim", "idx_heads", "idx_dim", "out_groups", "max_len", "dtype")


class _OShape(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in _FIELDS]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_n_vis.restype = ctypes.c_int32
        lib.oracle_n_vis.argtypes = [ctypes.c_int32, ctypes.c_int32]
        lib.oracle_select_row.restype = ctypes.c_int32
        lib.oracle_select_row.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p]
        lib.oracle_round_bf16.restype = ctypes.c_float
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_run.restype = ctypes.c_int32
        lib.oracle_swa_writeback.restype = None
        lib.oracle_swa_writeback.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_int32]
        lib.oracle_run.argtypes = ([ctypes.POINTER(_OShape)] + [ctypes.c_int32] * 4
                                   + [ctypes.c_void_p] * 13 + [ctypes.c_int32, ctypes.c_float,
                                                               ctypes.c_void_p, ctypes.c_void_p,
                                                               ctypes.c_void_p])
        _lib = lib
    return _lib


def n_vis(p: int, ratio: int) -> int:
    return int(_get().oracle_n_vis(int(p), int(ratio)))


def round_bf16(x: float) -> float:
    return float(_get().oracle_round_bf16(float(x)))


def e4m3_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 code, as the oracle decodes it."""
    return float(_get().oracle_e4m3_value(int(code)))


def swa_writeback(k_new: np.ndarray, v_new: np.ndarray, slot_mapping: np.ndarray,
                  k_cache: np.ndarray, v_cache: np.ndarray) -> tuple:
    """Copies of the caches after the writeback of rows k_new/v_new [T, D] to
    rows slot_mapping[t] of the caches [n_slots, D] (slots outside the cache
    are padding)."""
    kn, vn = np.ascontiguousarray(k_new), np.ascontiguousarray(v_new)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    kc, vc = np.ascontiguousarray(k_cache).copy(), np.ascontiguousarray(v_cache).copy()
    assert kn.shape == vn.shape and kc.shape == vc.shape and kn.shape[1] == kc.shape[1]
    assert kn.dtype == kc.dtype and sm.shape == (kn.shape[0],)
    _get().oracle_swa_writeback(kn.shape[0], kn.shape[1], kn.dtype.itemsize, kn.ctypes.data,
                                vn.ctypes.data, sm.ctypes.data, kc.ctypes.data, vc.ctypes.data,
                                kc.shape[0])
    return kc, vc


def select_row(scores: np.ndarray, k: int, n: Optional[int] = None) -> np.ndarray:
    s = np.ascontiguousarray(scores, dtype=np.float32)
    n = s.shape[0] if n is None else n
    out = np.empty(k, dtype=np.int32)
    rc = _get().oracle_select_row(s.ctypes.data, n, k, out.ctypes.data)
    if rc:
        raise RuntimeError(f"oracle_select_row failed ({rc})")
    return out


def unpage(pool: np.ndarray, block_table: np.ndarray, block_size: int, n_cap: int) -> np.ndarray:
    """Dense rows [B, n_cap, ...] of a paged cache: logical row j of request b
    is pool row block_table[b, j // block_size] * block_size + j % block_size
    (pool [n_blocks, block_size, ...])."""
    table = np.asarray(block_table, dtype=np.int64)
    j = np.arange(n_cap)
    phys = table[:, j // block_size] * block_size + j % block_size      # [B, n_cap]
    return pool.reshape(-1, *pool.shape[2:])[phys]


def run_paged(shape, inp: dict, **kw) -> dict:
    """The oracle on paged caches: the pools are first gathered to the dense
    per-request layout through the block tables, then `run` computes as usual.
    Paged names in `inp`: k_idx_pool (or k_idx8_pool + k_scale_pool) with
    idx_table / idx_block_size, k_cmp_pool + v_cmp_pool with cmp_table /
    cmp_block_size, and k_win_pool + v_win_pool with win_table /
    win_block_size (the window rings, logical row = ring slot)."""
    d = {k: v for k, v in inp.items() if not k.endswith(("_pool", "_table", "_block_size"))}
    nc = shape.n_cap
    if "k_idx_pool" in inp:
        d["k_idx"] = unpage(inp["k_idx_pool"], inp["idx_table"], inp["idx_block_size"], nc)
    if "k_idx8_pool" in inp:
        d["k_idx8"] = unpage(inp["k_idx8_pool"], inp["idx_table"], inp["idx_block_size"], nc)
        d["k_scale"] = unpage(inp["k_scale_pool"], inp["idx_table"], inp["idx_block_size"], nc)
    if "k_cmp_pool" in inp:
        d["k_cmp"] = unpage(inp["k_cmp_pool"], inp["cmp_table"], inp["cmp_block_size"], nc)
        d["v_cmp"] = unpage(inp["v_cmp_pool"], inp["cmp_table"], inp["cmp_block_size"], nc)
    if "k_win_pool" in inp:
        wc = shape.w_cap
        d["k_win"] = unpage(inp["k_win_pool"], inp["win_table"], inp["win_block_size"], wc)
        d["v_win"] = unpage(inp["v_win_pool"], inp["win_table"], inp["win_block_size"], wc)
    return run(shape, d, **kw)


def _ptr(a):
    return None if a is None else a.ctypes.data


def run(shape, inp: dict, jobs: int = JOB_SCORE | JOB_TOPK | JOB_ATTN, scale: Optional[float] = None,
        scores: Optional[np.ndarray] = None, topk_idx: Optional[np.ndarray] = None,
        tokens: Optional[tuple] = None, nthreads: int = 1) -> dict:
    """Run the chosen steps over tokens [t0, t1) (all tokens by default).

    `inp` is the dict from the seeded input generator.  `scores` / `topk_idx`
    may be given to start from a later step; otherwise they are allocated
    (scores filled with NaN, so untouched entries stay recognisable).  When
    `inp` holds "k_idx8" and "k_scale" (an FP8 indexer key cache), the keys
    come from those and "k_idx" is not read.
    Returns dict(scores, topk_idx, out) with out as float32 [G, B*S, (H/G)*D].
    """
    sh = _OShape(*[int(getattr(shape, f)) for f in _FIELDS])
    B, S, K, Nc = shape.batch, shape.q_per_req, shape.topk, shape.n_cap
    H, D, G = shape.heads, shape.head_dim, shape.out_groups
    if scores is None:
        scores = np.full((B, S, Nc), np.nan, dtype=np.float32)
    else:
        scores = np.ascontiguousarray(scores, dtype=np.float32).copy()
    if topk_idx is None:
        topk_idx = inp.get("topk_idx")
        topk_idx = (np.full((B, S, K), -7, dtype=np.int32) if topk_idx is None
                    else np.ascontiguousarray(topk_idx, np.int32).copy())
    else:
        topk_idx = np.ascontiguousarray(topk_idx, dtype=np.int32).copy()
    out = np.full((G, B * S, (H // G) * D), np.nan, dtype=np.float32)
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(D)))
    t0, t1 = (0, B * S) if tokens is None else tokens
    a = {k: (np.ascontiguousarray(v) if v is not None else None) for k, v in inp.items()}
    rc = _get().oracle_run(
        ctypes.byref(sh), int(jobs), int(t0), int(t1), int(nthreads),
        _ptr(a.get("q_idx")), _ptr(a.get("w")), _ptr(a.get("k_idx")), _ptr(a["start_pos"]),
        scores.ctypes.data, topk_idx.ctypes.data,
        _ptr(a.get("q")), _ptr(a.get("k_win")), _ptr(a.get("v_win")), _ptr(a.get("k_cmp")),
        _ptr(a.get("v_cmp")), _ptr(a.get("rope_cos")), _ptr(a.get("rope_sin")),
        int(a["rope_cos"].shape[0]) if a.get("rope_cos") is not None else 0,
        float(scale), out.ctypes.data, _ptr(a.get("k_idx8")), _ptr(a.get("k_scale")))
    if rc:
        raise RuntimeError(f"oracle_run failed with code {rc}")
    return dict(scores=scores, topk_idx=topk_idx, out=out)
