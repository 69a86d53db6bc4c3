"""Python binding of libcsa (ctypes).  Argument marshalling only.

Every function takes device tensors (torch, on a ROCm GPU), passes their
device pointers and sizes through the C ABI declared in include/csa.h and
raises if the library returns an error.  There is no CPU path: a missing
library, a CPU tensor or a non-contiguous tensor is an error.

Names match the C ABI: indexer_score, indexer_score_fp8,
indexer_score_paged, topk, sparse_attn_decode, sparse_attn_decode_paged,
sparse_attn_decode_noalloc, swa_writeback, plus the workspace queries and
step(), which issues the three calls in order on one stream.
"""
from __future__ import annotations

import ctypes
import functools
import os
from typing import Optional

import numpy as np
import torch

from .inputs import BF16, F32, Shape

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

_FIELDS = ("batch", "q_per_req", "ratio", "n_cap", "topk", "win", "w_cap", "heads",
           "head_dim", "rope_dim", "idx_heads", "idx_dim", "out_groups", "max_len", "dtype")

STATUS = {0: "CSA_OK", 1: "CSA_ERR_NULL_PTR", 2: "CSA_ERR_BAD_SHAPE", 3: "CSA_ERR_BAD_DTYPE",
          4: "CSA_ERR_CAPACITY", 5: "CSA_ERR_ALIGNMENT", 6: "CSA_ERR_WORKSPACE",
          7: "CSA_ERR_LAUNCH", 8: "CSA_ERR_UNSUPPORTED"}

# The argument lists below are those of this ABI version (CSA_ABI_VERSION).
ABI_VERSION = 2

EXPORTS = ("csa_indexer_score", "csa_indexer_score_fp8", "csa_indexer_score_paged",
           "csa_topk_workspace_bytes", "csa_topk", "csa_sparse_attn_workspace_bytes",
           "csa_sparse_attn_decode", "csa_sparse_attn_decode_paged",
           "csa_sparse_attn_decode_noalloc", "csa_sparse_attn_noalloc_max_workspace_bytes",
           "csa_swa_writeback", "csa_status_string", "csa_abi_version")


class CShape(ctypes.Structure):
    """Mirror of csa_shape_t."""
    _fields_ = [(f, ctypes.c_int32) for f in _FIELDS]

    @classmethod
    def of(cls, shape) -> "CShape":
        """The C struct of a shape (for a Shape, one struct per distinct shape,
        reused across calls: the library only reads it)."""
        if isinstance(shape, Shape):
            return _cshape_cached(shape)
        return cls(*[int(getattr(shape, f)) for f in _FIELDS])


@functools.lru_cache(maxsize=256)
def _cshape_cached(shape: Shape) -> CShape:
    return CShape(*[int(getattr(shape, f)) for f in _FIELDS])


class CPages(ctypes.Structure):
    """Mirror of csa_pages_t."""
    _fields_ = [("block_table", ctypes.c_void_p), ("blocks_per_req", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("n_blocks", ctypes.c_int64)]


class CsaError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({text})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcsa.so (built in-tree by build.py); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_attention_decode_csa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        sp = ctypes.POINTER(CShape)
        L.csa_indexer_score.restype = i32
        L.csa_indexer_score.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.csa_indexer_score_fp8.restype = i32
        L.csa_indexer_score_fp8.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
        pp = ctypes.POINTER(CPages)
        L.csa_indexer_score_paged.restype = i32
        L.csa_indexer_score_paged.argtypes = [sp, vp, vp, vp, vp, pp, vp, vp, vp]
        L.csa_sparse_attn_decode_paged.restype = i32
        L.csa_sparse_attn_decode_paged.argtypes = [sp, vp, vp, vp, vp, vp, pp, vp, vp, vp, vp, i32,
                                                   f32, vp, vp, sz, vp, pp]
        L.csa_topk_workspace_bytes.restype = sz
        L.csa_topk_workspace_bytes.argtypes = [sp]
        L.csa_topk.restype = i32
        L.csa_topk.argtypes = [sp, vp, vp, vp, vp, sz, vp]
        L.csa_sparse_attn_workspace_bytes.restype = sz
        L.csa_sparse_attn_workspace_bytes.argtypes = [sp]
        L.csa_sparse_attn_decode.restype = i32
        L.csa_sparse_attn_decode.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp,
                                             vp, sz, vp]
        L.csa_sparse_attn_decode_noalloc.restype = i32
        L.csa_sparse_attn_decode_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                                     f32, vp, vp]
        L.csa_sparse_attn_noalloc_max_workspace_bytes.restype = sz
        L.csa_sparse_attn_noalloc_max_workspace_bytes.argtypes = []
        L.csa_swa_writeback.restype = i32
        L.csa_swa_writeback.argtypes = [sp, vp, vp, vp, vp, vp, ctypes.c_int64, vp]
        L.csa_status_string.restype = ctypes.c_char_p
        L.csa_status_string.argtypes = [i32]
        L.csa_abi_version.restype = i32
        L.csa_abi_version.argtypes = []
        got = L.csa_abi_version()
        if got != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} implements ABI version {got}, this binding expects "
                              f"{ABI_VERSION}: rebuild it with "
                              "`python -m sparse_attention_decode_csa_amd.build`")
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().csa_status_string(int(code)).decode()


def _check(fn: str, code: int):
    if code != 0:
        raise CsaError(fn, code, status_string(code))


def _dev(t: Optional[torch.Tensor], name: str, numel: Optional[int] = None,
         dtype: Optional[torch.dtype] = None, esize: Optional[int] = None):
    """Device pointer of a contiguous GPU tensor (None -> NULL).

    The C ABI takes pointers only, so a tensor smaller than the shape implies
    would be read or written past its end on the device: with `numel` the
    tensor must hold at least that many elements, with `dtype` exactly that
    element type, with `esize` elements of that many bytes (for copies, which
    take any type of the right width)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: tensor must live on the GPU (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if esize is not None and t.element_size() != esize:
        raise TypeError(f"{name}: expected {esize}-byte elements, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name}: {t.numel()} elements, the shape needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        # the current stream's raw handle without building a Stream object
        # (several microseconds per call otherwise)
        try:
            return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()))
        except AttributeError:
            stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def torch_dtype(shape) -> torch.dtype:
    return torch.bfloat16 if shape.dtype == BF16 else torch.float32


def topk_workspace_bytes(shape) -> int:
    return int(lib().csa_topk_workspace_bytes(ctypes.byref(CShape.of(shape))))


def sparse_attn_workspace_bytes(shape) -> int:
    return int(lib().csa_sparse_attn_workspace_bytes(ctypes.byref(CShape.of(shape))))


def _sizes(shape) -> dict:
    """Element counts the shape implies for each tensor of the step."""
    if isinstance(shape, Shape):
        return _sizes_cached(shape)
    return _sizes_of(shape)


@functools.lru_cache(maxsize=256)
def _sizes_cached(shape: Shape) -> dict:
    return _sizes_of(shape)


def _sizes_of(shape) -> dict:
    B, S, Hi, Di = shape.batch, shape.q_per_req, shape.idx_heads, shape.idx_dim
    return dict(q_idx=B * S * Hi * Di, w=B * S * Hi, k_idx=B * shape.n_cap * Di, start_pos=B,
                scores=B * S * shape.n_cap, topk_idx=B * S * shape.topk,
                q=B * S * shape.heads * shape.head_dim, win=B * shape.w_cap * shape.head_dim,
                cmp=B * shape.n_cap * shape.head_dim, k_scale=B * shape.n_cap)


def indexer_score(shape, q_idx, w, k_idx, start_pos, scores, stream=None) -> None:
    cs, n, dt = CShape.of(shape), _sizes(shape), torch_dtype(shape)
    _check("csa_indexer_score", lib().csa_indexer_score(
        ctypes.byref(cs), _dev(q_idx, "q_idx", n["q_idx"], dt), _dev(w, "w", n["w"], torch.float32),
        _dev(k_idx, "k_idx", n["k_idx"], dt), _dev(start_pos, "start_pos", n["start_pos"], torch.int32),
        _dev(scores, "scores", n["scores"], torch.float32), _stream(stream)))


def indexer_score_fp8(shape, q_idx, w, k_idx8, k_scale, start_pos, scores, stream=None) -> None:
    cs, n = CShape.of(shape), _sizes(shape)
    _check("csa_indexer_score_fp8", lib().csa_indexer_score_fp8(
        ctypes.byref(cs), _dev(q_idx, "q_idx", n["q_idx"], torch.bfloat16),
        _dev(w, "w", n["w"], torch.float32), _dev(k_idx8, "k_idx8", n["k_idx"], torch.uint8),
        _dev(k_scale, "k_scale", n["k_scale"], torch.float32),
        _dev(start_pos, "start_pos", n["start_pos"], torch.int32),
        _dev(scores, "scores", n["scores"], torch.float32), _stream(stream)))


def _pages(shape, pool, block_table, name: str, row: int) -> CPages:
    """csa_pages_t of a pool [n_blocks, block_size, row] and its table [B, blocks_per_req]."""
    if pool.dim() < 2 or block_table.dim() != 2 or block_table.dtype != torch.int32:
        raise ValueError(f"{name}: pool [n_blocks, block_size, ...] and int32 table [B, bpr] expected")
    if pool.shape[2:].numel() != row:
        raise ValueError(f"{name}: pool rows of {pool.shape[2:].numel()} elements, the shape needs {row}")
    if block_table.shape[0] < shape.batch:
        raise ValueError(f"{name}: block table has {block_table.shape[0]} rows for {shape.batch} requests")
    return CPages(_dev(block_table, name + " block_table"), int(block_table.shape[1]),
                  int(pool.shape[1]), int(pool.shape[0]))


def indexer_score_paged(shape, q_idx, w, k_pool, k_scale, block_table, start_pos, scores,
                        stream=None) -> None:
    """k_pool [n_blocks, block_size, Di] (shape.dtype keys, or uint8 E4M3 codes
    with k_scale [n_blocks, block_size] float32); block_table [B, bpr] int32."""
    cs, n, dt = CShape.of(shape), _sizes(shape), torch_dtype(shape)
    pg = _pages(shape, k_pool, block_table, "k_pool", shape.idx_dim)
    rows = pg.n_blocks * pg.block_size
    kdt = torch.uint8 if k_scale is not None else dt
    _check("csa_indexer_score_paged", lib().csa_indexer_score_paged(
        ctypes.byref(cs), _dev(q_idx, "q_idx", n["q_idx"], torch.bfloat16 if k_scale is not None else dt),
        _dev(w, "w", n["w"], torch.float32), _dev(k_pool, "k_pool", rows * shape.idx_dim, kdt),
        _dev(k_scale, "k_scale", rows, torch.float32), ctypes.byref(pg),
        _dev(start_pos, "start_pos", n["start_pos"], torch.int32),
        _dev(scores, "scores", n["scores"], torch.float32), _stream(stream)))


def topk(shape, scores, start_pos, topk_idx, ws=None, stream=None) -> None:
    cs, n = CShape.of(shape), _sizes(shape)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa_topk", lib().csa_topk(
        ctypes.byref(cs), _dev(scores, "scores", n["scores"], torch.float32),
        _dev(start_pos, "start_pos", n["start_pos"], torch.int32),
        _dev(topk_idx, "topk_idx", n["topk_idx"], torch.int32), _dev(ws, "ws"), nbytes,
        _stream(stream)))


def _attn_common(shape, q, k_win, v_win, topk_idx, start_pos, rope_cos, rope_sin, out,
                 win_numel=None):
    """Pointers of the arguments both attention entries share, size-checked
    (win_numel: elements of a paged window pool instead of the dense rings)."""
    n, dt = _sizes(shape), torch_dtype(shape)
    nw = n["win"] if win_numel is None else win_numel
    rope_rows = 0 if rope_cos is None else int(rope_cos.shape[0])
    half = shape.rope_dim // 2
    for name, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
        # rows of Dr/2 pairs, one row per position
        if t is not None and (t.dim() != 2 or t.shape[1] != half or t.shape[0] != rope_rows):
            raise ValueError(f"{name}: expected [{rope_rows or 'rows'}, {half}], got {list(t.shape)}")
    return dict(q=_dev(q, "q", n["q"], dt), k_win=_dev(k_win, "k_win", nw, dt),
                v_win=_dev(v_win, "v_win", nw, dt),
                topk_idx=_dev(topk_idx, "topk_idx", n["topk_idx"], torch.int32),
                start_pos=_dev(start_pos, "start_pos", n["start_pos"], torch.int32),
                rope_cos=_dev(rope_cos, "rope_cos", rope_rows * half, torch.float32),
                rope_sin=_dev(rope_sin, "rope_sin", rope_rows * half, torch.float32),
                rope_rows=rope_rows, out=_dev(out, "out", n["q"], dt))


def sparse_attn_decode(shape, q, k_win, v_win, k_cmp, v_cmp, topk_idx, start_pos, rope_cos,
                       rope_sin, softmax_scale, out, ws, stream=None) -> None:
    cs, n, dt = CShape.of(shape), _sizes(shape), torch_dtype(shape)
    c = _attn_common(shape, q, k_win, v_win, topk_idx, start_pos, rope_cos, rope_sin, out)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa_sparse_attn_decode", lib().csa_sparse_attn_decode(
        ctypes.byref(cs), c["q"], c["k_win"], c["v_win"], _dev(k_cmp, "k_cmp", n["cmp"], dt),
        _dev(v_cmp, "v_cmp", n["cmp"], dt), c["topk_idx"], c["start_pos"], c["rope_cos"],
        c["rope_sin"], c["rope_rows"], float(softmax_scale), c["out"], _dev(ws, "ws"), nbytes,
        _stream(stream)))


def sparse_attn_decode_noalloc(shape, q, k_win, v_win, k_cmp, v_cmp, topk_idx, start_pos,
                               rope_cos, rope_sin, softmax_scale, out, stream=None) -> None:
    """sparse_attn_decode without a workspace: the split partials live in the
    library's static device array (see csa_sparse_attn_noalloc_max_workspace_bytes)."""
    cs, n, dt = CShape.of(shape), _sizes(shape), torch_dtype(shape)
    c = _attn_common(shape, q, k_win, v_win, topk_idx, start_pos, rope_cos, rope_sin, out)
    _check("csa_sparse_attn_decode_noalloc", lib().csa_sparse_attn_decode_noalloc(
        ctypes.byref(cs), c["q"], c["k_win"], c["v_win"], _dev(k_cmp, "k_cmp", n["cmp"], dt),
        _dev(v_cmp, "v_cmp", n["cmp"], dt), c["topk_idx"], c["start_pos"], c["rope_cos"],
        c["rope_sin"], c["rope_rows"], float(softmax_scale), c["out"], _stream(stream)))


def sparse_attn_noalloc_max_workspace_bytes() -> int:
    return int(lib().csa_sparse_attn_noalloc_max_workspace_bytes())


def sparse_attn_decode_paged(shape, q, k_win, v_win, k_pool, v_pool, block_table, topk_idx,
                             start_pos, rope_cos, rope_sin, softmax_scale, out, ws,
                             stream=None, win_table=None) -> None:
    """k_pool/v_pool [n_blocks, block_size, D] sharing block_table [B, bpr] int32.
    With win_table [B, wbpr] int32, k_win/v_win are pools [n_blocks, block_size, D]
    of the window rings as well (ring slot r of request b is pool row
    win_table[b, r // block_size] * block_size + r % block_size)."""
    cs, dt = CShape.of(shape), torch_dtype(shape)
    if k_pool.shape != v_pool.shape:
        raise ValueError("k_pool and v_pool must have the same shape")
    pg = _pages(shape, k_pool, block_table, "k_pool", shape.head_dim)
    rows = pg.n_blocks * pg.block_size
    wpg, win_numel = None, None
    if win_table is not None:
        if k_win.shape != v_win.shape:
            raise ValueError("k_win and v_win pools must have the same shape")
        wpg = _pages(shape, k_win, win_table, "k_win", shape.head_dim)
        win_numel = wpg.n_blocks * wpg.block_size * shape.head_dim
    c = _attn_common(shape, q, k_win, v_win, topk_idx, start_pos, rope_cos, rope_sin, out, win_numel)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa_sparse_attn_decode_paged", lib().csa_sparse_attn_decode_paged(
        ctypes.byref(cs), c["q"], c["k_win"], c["v_win"],
        _dev(k_pool, "k_pool", rows * shape.head_dim, dt), _dev(v_pool, "v_pool", rows * shape.head_dim, dt),
        ctypes.byref(pg), c["topk_idx"], c["start_pos"], c["rope_cos"], c["rope_sin"],
        c["rope_rows"], float(softmax_scale), c["out"], _dev(ws, "ws"), nbytes, _stream(stream),
        None if wpg is None else ctypes.byref(wpg)))


def swa_writeback(shape, k_new, v_new, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """k_new/v_new [B*S, D]; k_cache/v_cache [n_slots, D] (any leading shape
    whose rows are D elements, e.g. the [B, w_cap, D] rings)."""
    cs = CShape.of(shape)
    es = 2 if shape.dtype == BF16 else 4  # a row copy: any element type of that width
    if k_cache.numel() != v_cache.numel():
        raise ValueError("k_cache and v_cache must hold the same number of rows")
    n_slots = k_cache.numel() // shape.head_dim
    T = shape.batch * shape.q_per_req
    _check("csa_swa_writeback", lib().csa_swa_writeback(
        ctypes.byref(cs), _dev(k_new, "k_new", T * shape.head_dim, esize=es),
        _dev(v_new, "v_new", T * shape.head_dim, esize=es),
        _dev(slot_mapping, "slot_mapping", T, torch.int32), _dev(k_cache, "k_cache", esize=es),
        _dev(v_cache, "v_cache", esize=es), n_slots, _stream(stream)))


# ----------------------------------------------------------------------------
# convenience: device buffers for one step
# ----------------------------------------------------------------------------

def to_device(inp: dict, shape, device="cuda") -> dict:
    """Upload a seeded input dict: bf16 bit patterns become torch.bfloat16;
    plain numbers (block sizes) are left out."""
    out = {}
    for k, v in inp.items():
        if not isinstance(v, np.ndarray):
            continue
        if v.dtype == np.uint16:
            t = torch.from_numpy(v.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(v))
        out[k] = t.to(device, non_blocking=False).contiguous()
    return out


def alloc_topk_workspace(shape, device="cuda") -> Optional[torch.Tensor]:
    """The workspace csa_topk needs for this shape (None when it needs none)."""
    n = topk_workspace_bytes(shape)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def alloc_outputs(shape, device="cuda", scores_fill=float("nan")) -> dict:
    """Output and workspace buffers of one step."""
    B, S, Nc, K = shape.batch, shape.q_per_req, shape.n_cap, shape.topk
    G, H, D = shape.out_groups, shape.heads, shape.head_dim
    dt = torch_dtype(shape)
    aw = sparse_attn_workspace_bytes(shape)
    return dict(
        scores=torch.full((B, S, Nc), scores_fill, dtype=torch.float32, device=device),
        topk_idx=torch.full((B, S, K), -7, dtype=torch.int32, device=device),
        out=torch.empty((G, B * S, (H // G) * D), dtype=dt, device=device),
        topk_ws=alloc_topk_workspace(shape, device),
        attn_ws=torch.empty(max(aw, 16), dtype=torch.uint8, device=device),
    )


def step(shape, dev: dict, bufs: dict, softmax_scale: float, stream=None,
         supplied_topk: bool = False) -> None:
    """One decode step: score, select, attend (or attend only, when the
    caller supplies the Top-K lists in dev['topk_idx'])."""
    if supplied_topk:
        ti = dev["topk_idx"]
    else:
        if "idx_table" in dev:   # paged indexer key cache (bf16/f32 keys or FP8 codes)
            fp8 = "k_idx8_pool" in dev
            indexer_score_paged(shape, dev["q_idx"], dev["w"],
                                dev["k_idx8_pool"] if fp8 else dev["k_idx_pool"],
                                dev["k_scale_pool"] if fp8 else None, dev["idx_table"],
                                dev["start_pos"], bufs["scores"], stream)
        elif "k_idx8" in dev:   # FP8 indexer key cache
            indexer_score_fp8(shape, dev["q_idx"], dev["w"], dev["k_idx8"], dev["k_scale"],
                              dev["start_pos"], bufs["scores"], stream)
        else:
            indexer_score(shape, dev["q_idx"], dev["w"], dev["k_idx"], dev["start_pos"],
                          bufs["scores"], stream)
        topk(shape, bufs["scores"], dev["start_pos"], bufs["topk_idx"], bufs["topk_ws"], stream)
        ti = bufs["topk_idx"]
    if "cmp_table" in dev:   # paged compressed K/V cache (and maybe paged window rings)
        paged_win = "win_table" in dev
        sparse_attn_decode_paged(shape, dev["q"], dev["k_win_pool" if paged_win else "k_win"],
                                 dev["v_win_pool" if paged_win else "v_win"], dev["k_cmp_pool"],
                                 dev["v_cmp_pool"], dev["cmp_table"], ti, dev["start_pos"],
                                 dev["rope_cos"], dev["rope_sin"], softmax_scale, bufs["out"],
                                 bufs["attn_ws"], stream, dev.get("win_table"))
        return
    sparse_attn_decode(shape, dev["q"], dev["k_win"], dev["v_win"], dev["k_cmp"], dev["v_cmp"],
                       ti, dev["start_pos"], dev["rope_cos"], dev["rope_sin"], softmax_scale,
                       bufs["out"], bufs["attn_ws"], stream)
