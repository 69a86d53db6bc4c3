"""The C-ABI library on the CPU: it loads, exports what include/csa.h declares,
and its host-side checks refuse bad arguments before any GPU work.

No call here reaches a kernel launch: every call is refused by validation (or
is the empty problem, which returns before touching the GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_attention_decode_csa_amd import csa as C
from sparse_attention_decode_csa_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced (calls are refused first)
MISALIGNED = ctypes.c_void_p(0x10004)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(csa_\w+)\s*\(", text, flags=re.M)))


def test_header_and_exports_agree():
    decl = declared_functions()
    assert set(decl) == set(C.EXPORTS), decl
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (csa_\w+)", out))
    assert set(decl) <= exported, set(decl) - exported
    lib = C.lib()
    for name in decl:
        assert hasattr(lib, name)


def test_version_and_status_strings():
    header_version = int(re.search(r"#define CSA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert C.lib().csa_abi_version() == C.ABI_VERSION == header_version
    for code in range(9):
        assert C.status_string(code)
    assert C.status_string(99) == "unknown status"


def shape(**kw):
    return I.CONFIGS[1].shape.replace(**kw)


def call_score(sh, ptrs=None):
    p = ptrs or [FAKE] * 5
    return C.lib().csa_indexer_score(None if sh is None else ctypes.byref(C.CShape.of(sh)),
                                     *p, None)


def call_topk(sh, ptrs=None):
    p = ptrs or [FAKE] * 3
    return C.lib().csa_topk(ctypes.byref(C.CShape.of(sh)), *p, None, 0, None)


def call_attn(sh, ptrs=None, rope_rows=1 << 20, ws_bytes=1 << 40, scale=0.1):
    p = ptrs or [FAKE] * 10
    return C.lib().csa_sparse_attn_decode(ctypes.byref(C.CShape.of(sh)), *p[:9], rope_rows, scale,
                                          p[9], FAKE, ws_bytes, None)


@pytest.mark.parametrize("case,code", [
    (dict(dtype=5), 3),
    (dict(batch=-1), 2),
    (dict(ratio=0), 2),
    (dict(topk=0), 2),
    (dict(topk=5000), 8),
    (dict(idx_dim=96), 8),
    (dict(idx_heads=65), 8),
    (dict(n_cap=200), 4),            # floor(1024 / 4) = 256 rows needed
    (dict(max_len=0), 2),
])
def test_indexer_score_refusals(case, code):
    assert call_score(shape(**case)) == code


def test_indexer_score_null_and_alignment():
    assert call_score(None) == 1
    assert call_score(shape(), [FAKE, None, FAKE, FAKE, FAKE]) == 1
    assert call_score(shape(), [FAKE, FAKE, MISALIGNED, FAKE, FAKE]) == 5


def call_score_fp8(sh, ptrs=None):
    p = ptrs or [FAKE] * 6
    return C.lib().csa_indexer_score_fp8(None if sh is None else ctypes.byref(C.CShape.of(sh)),
                                         *p, None)


@pytest.mark.parametrize("case,code", [
    (dict(dtype=I.F32), 3),          # bf16 queries only
    (dict(dtype=5), 3),
    (dict(idx_dim=96), 8),
    (dict(idx_heads=65), 8),
    (dict(n_cap=200), 4),
    (dict(batch=-1), 2),
])
def test_indexer_score_fp8_refusals(case, code):
    assert call_score_fp8(shape(**case)) == code


def test_indexer_score_fp8_null_and_alignment():
    assert call_score_fp8(None) == 1
    assert call_score_fp8(shape(), [FAKE, FAKE, FAKE, None, FAKE, FAKE]) == 1   # k_scale
    assert call_score_fp8(shape(), [FAKE, FAKE, None, FAKE, FAKE, FAKE]) == 1   # codes
    assert call_score_fp8(shape(), [FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE]) == 5
    assert call_score_fp8(shape(batch=0), [None] * 6) == 0  # empty problem


def call_writeback(sh, ptrs=None, n_slots=100):
    p = ptrs or [FAKE] * 5
    return C.lib().csa_swa_writeback(None if sh is None else ctypes.byref(C.CShape.of(sh)),
                                     *p, n_slots, None)


@pytest.mark.parametrize("case,n_slots,code", [
    (dict(dtype=5), 100, 3),
    (dict(batch=-1), 100, 2),
    (dict(head_dim=0), 100, 2),
    (dict(), -1, 2),
    (dict(head_dim=6), 100, 8),               # 12-byte bf16 rows: not whole 16-byte pieces
    (dict(head_dim=6, dtype=I.F32), 100, 8),  # 24-byte rows
])
def test_writeback_refusals(case, n_slots, code):
    assert call_writeback(shape(**case), n_slots=n_slots) == code


def test_writeback_null_alignment_empty():
    assert call_writeback(None) == 1
    assert call_writeback(shape(), [FAKE, FAKE, None, FAKE, FAKE]) == 1
    assert call_writeback(shape(), [FAKE, FAKE, FAKE, MISALIGNED, FAKE]) == 5
    assert call_writeback(shape(q_per_req=0), [None] * 5) == 0
    assert call_writeback(shape(head_dim=4, dtype=I.F32), [FAKE] * 4 + [MISALIGNED]) == 5


@pytest.mark.parametrize("case,code", [
    (dict(n_cap=255), 4),
    (dict(win=0), 2),
    (dict(dtype=-1), 3),
])
def test_topk_refusals(case, code):
    assert call_topk(shape(**case)) == code


def test_topk_null():
    assert call_topk(shape(), [FAKE, None, FAKE]) == 1


def test_topk_workspace_refusals():
    # rows past 32768 keys are split over several workgroups, whose
    # candidates need the workspace
    sh = I.CONFIGS[3].shape.replace(n_cap=65536, max_len=4 * 65536)
    need = C.topk_workspace_bytes(sh)
    assert need > 0
    lib = C.lib()
    cs = ctypes.byref(C.CShape.of(sh))
    assert lib.csa_topk(cs, FAKE, FAKE, FAKE, None, 0, None) == 6
    assert lib.csa_topk(cs, FAKE, FAKE, FAKE, FAKE, need - 1, None) == 6
    assert lib.csa_topk(cs, FAKE, FAKE, FAKE, MISALIGNED, need, None) == 5


@pytest.mark.parametrize("case,code", [
    (dict(head_dim=96, rope_dim=32), 8),
    (dict(heads=65), 8),
    (dict(rope_dim=63), 2),
    (dict(rope_dim=256), 2),
    (dict(heads=16, out_groups=3), 2),
    (dict(w_cap=127), 4),            # needs win + S - 1 = 128
    (dict(q_per_req=2, w_cap=128), 4),
])
def test_attn_refusals(case, code):
    assert call_attn(shape(**case)) == code


def split_shape(**kw):
    """A shape whose window and Top-K rows do not fit one workgroup per token:
    the split kernels and their workspace."""
    return shape(topk=1024, **kw)


def test_attn_capacity_workspace_alignment():
    sh = shape()
    assert call_attn(sh, rope_rows=1000) == 4            # max_len = 1024 rows needed
    sp = split_shape()
    assert call_attn(sp, ws_bytes=C.sparse_attn_workspace_bytes(sp) - 1) == 6
    assert call_attn(sh, scale=float("nan")) == 2
    p = [FAKE] * 10
    p[2] = MISALIGNED
    assert call_attn(sh, p) == 5
    p = [FAKE] * 10
    p[0] = None
    assert call_attn(sh, p) == 1
    p = [FAKE] * 10
    p[7] = None                                          # rope table with rope_dim > 0
    assert call_attn(sh, p) == 1
    # no RoPE: NULL tables pass the pointer checks (refused later, for the workspace)
    assert call_attn(split_shape(rope_dim=0), [FAKE] * 7 + [None, None, FAKE], ws_bytes=0) == 6


def call_attn_noalloc(sh, ptrs=None, rope_rows=1 << 20, scale=0.1):
    p = ptrs or [FAKE] * 10
    return C.lib().csa_sparse_attn_decode_noalloc(ctypes.byref(C.CShape.of(sh)), *p[:9], rope_rows,
                                                  scale, p[9], None)


def test_attn_noalloc_refusals():
    # Every check runs before the static array is looked up on the device, so
    # these refusals need no GPU.
    cap = C.sparse_attn_noalloc_max_workspace_bytes()
    assert cap == 32 << 20
    sh = shape()
    assert C.sparse_attn_workspace_bytes(sh) <= cap
    assert call_attn_noalloc(sh, rope_rows=1000) == 4
    assert call_attn_noalloc(shape(w_cap=127)) == 4
    assert call_attn_noalloc(shape(heads=65)) == 8
    assert call_attn_noalloc(sh, scale=float("inf")) == 2
    p = [FAKE] * 10
    p[9] = MISALIGNED
    assert call_attn_noalloc(sh, p) == 5
    p = [FAKE] * 10
    p[4] = None
    assert call_attn_noalloc(sh, p) == 1
    # a shape whose split partials exceed the static array
    big = shape(batch=4096, topk=4096, win=4096, w_cap=4096, max_len=1024)
    assert C.sparse_attn_workspace_bytes(big) > cap
    assert call_attn_noalloc(big) == 6
    assert call_attn_noalloc(shape(batch=0)) == 0


def test_empty_problem_is_ok_without_gpu_work():
    sh = shape(batch=0)
    assert call_score(sh) == 0 and call_topk(sh) == 0 and call_attn(sh) == 0
    assert C.sparse_attn_workspace_bytes(sh) == 0


def test_workspace_queries():
    for cid, cfg in I.CONFIGS.items():
        sh = cfg.shape
        # rows of at most 32768 keys: one workgroup per row, no workspace
        assert C.topk_workspace_bytes(sh) == 0, cid
        ws = C.sparse_attn_workspace_bytes(sh)
        T = sh.batch * sh.q_per_req
        if cid == 2:
            # 128 tokens of 12 waves, one workgroup per token: no partials
            assert ws == 0, cid
        else:
            assert ws >= T * 2 * sh.heads * (sh.head_dim + 2) * 4, cid  # a split per stream at least
    # decode launches over longer rows select in two passes: a candidate slot
    # of a whole chunk per (token, chunk), and counts
    long = I.CONFIGS[4].shape.replace(n_cap=131072, max_len=4 * 131072)
    assert C.topk_workspace_bytes(long) >= long.batch * long.q_per_req * 131072 * 8


def test_binding_refuses_cpu_tensors():
    import torch
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        C.topk(shape(), t, t, t)


def test_binding_refuses_rope_tables_of_the_wrong_layout():
    # the tables hold Dr/2 (cos, sin) pairs per position; a full-width table
    # or mismatched row counts would be read with the wrong stride
    import torch
    sh = shape()
    t = torch.zeros(4)
    half = sh.rope_dim // 2
    for cos, sin in ((torch.zeros(sh.max_len, sh.rope_dim), torch.zeros(sh.max_len, half)),
                     (torch.zeros(sh.max_len, half), torch.zeros(sh.max_len - 1, half)),
                     (torch.zeros(sh.max_len * half), torch.zeros(sh.max_len * half))):
        with pytest.raises(ValueError, match="rope_"):
            C.sparse_attn_decode(sh, t, t, t, t, t, t, t, cos, sin, 0.1, t, t)


def test_binding_refuses_pools_of_the_wrong_row_width():
    # pool rows are read at a stride of Di (indexer) or D (attention) elements
    import torch
    sh = shape()
    t = torch.zeros(4)
    table = torch.zeros(sh.batch, 64, dtype=torch.int32)
    with pytest.raises(ValueError, match="pool rows"):
        C.indexer_score_paged(sh, t, t, torch.zeros(8, 16, sh.idx_dim + 8), None, table, t, t)
    bad = torch.zeros(8, 16, sh.head_dim // 2)
    with pytest.raises(ValueError, match="pool rows"):
        C.sparse_attn_decode_paged(sh, t, t, t, bad, bad, table, t, t, None, None, 0.1, t, t)


# --------------------------------------------------------------------------
# paged compressed caches
# --------------------------------------------------------------------------

def pages(bpr=16, bs=16, n_blocks=1000, table=FAKE):
    return C.CPages(table, bpr, bs, n_blocks)


def call_score_paged(sh, pg, ptrs=None, k_scale=None):
    p = ptrs or [FAKE] * 5
    return C.lib().csa_indexer_score_paged(
        None if sh is None else ctypes.byref(C.CShape.of(sh)), p[0], p[1], p[2], k_scale,
        None if pg is None else ctypes.byref(pg), p[3], p[4], None)


def call_attn_paged(sh, pg, ptrs=None, ws_bytes=1 << 40, win_pg=None):
    p = ptrs or [FAKE] * 10
    return C.lib().csa_sparse_attn_decode_paged(
        ctypes.byref(C.CShape.of(sh)), p[0], p[1], p[2], p[3], p[4],
        None if pg is None else ctypes.byref(pg), p[5], p[6], p[7], p[8], 1 << 20, 0.1, p[9],
        FAKE, ws_bytes, None, None if win_pg is None else ctypes.byref(win_pg))


# shape(): n_cap 256 rows, so block size 16 needs 16 table entries per request
PAGE_REFUSALS = [
    (dict(bs=8), 2), (dict(bs=48), 2), (dict(bs=8192), 2), (dict(bs=0), 2),
    (dict(n_blocks=0), 2), (dict(bpr=0), 2),
    (dict(bpr=15), 4), (dict(bpr=1, bs=128), 4),
    (dict(n_blocks=1 << 28, bs=16), 8),          # 2^32 pool rows: past int32
    (dict(n_blocks=(1 << 62) + 1, bs=4096), 8),   # rows x bytes would overflow int64
    (dict(table=MISALIGNED), 5), (dict(table=None), 1),
]


@pytest.mark.parametrize("kw,code", PAGE_REFUSALS)
def test_indexer_score_paged_refusals(kw, code):
    assert call_score_paged(shape(), pages(**kw)) == code


@pytest.mark.parametrize("kw,code", PAGE_REFUSALS + [
    (dict(n_blocks=(1 << 31) // (16 * 256), bs=16), 8),   # bf16 D=128 pool reaching 2^31 bytes
])
def test_attn_paged_refusals(kw, code):
    assert call_attn_paged(shape(), pages(**kw)) == code


# window rings paged: the csa_pages_t rules of the compressed pool, with the
# capacity taken against w_cap (shape(): w_cap 128, so 16-row blocks need 8)
@pytest.mark.parametrize("kw,code", [
    (dict(bs=8), 2), (dict(bs=48), 2), (dict(bs=8192), 2), (dict(bs=0), 2),
    (dict(n_blocks=0), 2), (dict(bpr=0), 2),
    (dict(bpr=7), 4), (dict(bpr=1, bs=64), 4),
    (dict(n_blocks=1 << 28, bs=16), 8),
    (dict(n_blocks=(1 << 31) // (16 * 256), bs=16), 8),   # bf16 D=128 pool reaching 2^31 bytes
    (dict(table=MISALIGNED), 5), (dict(table=None), 1),
])
def test_attn_paged_window_refusals(kw, code):
    sh = shape()
    assert sh.w_cap == 128
    assert call_attn_paged(sh, pages(), win_pg=pages(**kw)) == code


def test_attn_paged_window_tables_that_fit():
    sh = shape()
    # a window table covering exactly w_cap rows passes the page checks (the
    # call then stops at the missing workspace, before any launch)
    sp = split_shape()
    assert call_attn_paged(sp, pages(), ws_bytes=0, win_pg=pages(bpr=8, bs=16)) == 6
    assert call_attn_paged(sp, pages(), ws_bytes=0, win_pg=pages(bpr=1, bs=128)) == 6


def test_paged_null_dtype_alignment_workspace():
    assert call_score_paged(None, pages()) == 1
    assert call_score_paged(shape(), None) == 1
    assert call_score_paged(shape(), pages(), [FAKE, FAKE, None, FAKE, FAKE]) == 1   # pool
    assert call_score_paged(shape(), pages(), [FAKE, FAKE, MISALIGNED, FAKE, FAKE]) == 5
    assert call_score_paged(shape(dtype=I.F32), pages(), k_scale=FAKE) == 3         # FP8: bf16 q
    assert call_score_paged(shape(), pages(), k_scale=MISALIGNED) == 5
    assert call_score_paged(shape(n_cap=200), pages()) == 4     # capacity for max_len first
    assert call_score_paged(shape(batch=0), None, [None] * 5) == 0   # empty problem
    assert call_attn_paged(shape(), None) == 1
    p = [FAKE] * 10
    p[3] = None                                                  # k_pool
    assert call_attn_paged(shape(), pages(), p) == 1
    p = [FAKE] * 10
    p[4] = MISALIGNED                                            # v_pool
    assert call_attn_paged(shape(), pages(), p) == 5
    sh = split_shape()
    assert call_attn_paged(sh, pages(), ws_bytes=C.sparse_attn_workspace_bytes(sh) - 1) == 6
    # the largest pool the 32-bit offsets allow passes the page checks
    assert call_attn_paged(sh, pages(n_blocks=(0x7FFFF000 // (16 * 256))), ws_bytes=0) == 6
