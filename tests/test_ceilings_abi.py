"""The ceiling probes' library (libcsa_ceilings.so) on the CPU: it loads,
exports what include/csa_ceilings.h declares, and refuses bad arguments before
any launch.  No call here reaches a kernel."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa_ceilings.h")

import bench_ceilings as BC  # noqa: E402

FAKE = 0x10000       # aligned, never dereferenced (every call below is refused first)
MISALIGNED = 0x10004


@pytest.fixture(scope="module")
def P():
    return BC.load_ceilings()


def test_header_and_exports_agree(P):
    text = open(HEADER).read()
    decl = sorted(set(re.findall(r"^\s*int\s+(csa_ceiling_\w+)\s*\(", text, flags=re.M)))
    assert decl == ["csa_ceiling_gather", "csa_ceiling_stream_dma", "csa_ceiling_stream_vec"]
    out = subprocess.run(["nm", "-D", "--defined-only", BC.CEILINGS_LIB], capture_output=True,
                         text=True, check=True).stdout
    assert set(decl) <= set(re.findall(r"\bT (csa_\w+)", out))
    for name in decl:
        assert hasattr(P, name)
    # the constants the driver relies on are the header's
    assert int(re.search(r"CSA_CEILING_DMA_WG_BYTES (\d+)", text).group(1)) == BC.DMA_WG_BYTES
    assert int(re.search(r"CSA_CEILING_DMA_PAGE_BYTES (\d+)", text).group(1)) == BC.DMA_PAGE_BYTES


def test_decode_library_does_not_export_the_probes():
    from sparse_attention_decode_csa_amd import csa as C
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert "csa_ceiling" not in out


@pytest.mark.parametrize("args", [
    (None, 131072, None, 0, FAKE),            # null source
    (FAKE, 131072, None, 0, None),            # null sink
    (FAKE, 0, None, 0, FAKE),                 # empty
    (FAKE, 131072 + 16, None, 0, FAKE),       # not a whole number of workgroups
    (MISALIGNED, 131072, None, 0, FAKE),      # misaligned source
    (FAKE, 131072, FAKE, 0, FAKE),            # a page table over an empty pool
])
def test_stream_dma_refusals(P, args):
    assert P.csa_ceiling_stream_dma(*args, None) == -1


@pytest.mark.parametrize("args", [
    (None, 4096, 1024, 256, FAKE),
    (FAKE, 4096, 0, 256, FAKE),
    (FAKE, 4096, 1000, 256, FAKE),            # not a multiple of 16
    (FAKE, 4096, 3072, 256, FAKE),            # does not divide the size
    (FAKE, 4096, 1024, 512, FAKE),            # unsupported workgroup size
    (MISALIGNED, 4096, 1024, 256, FAKE),
])
def test_stream_vec_refusals(P, args):
    assert P.csa_ceiling_stream_vec(*args, None) == -1


@pytest.mark.parametrize("args", [
    (FAKE, FAKE, 1 << 20, FAKE, 0, FAKE),     # no rows
    (FAKE, FAKE, 1000, FAKE, 4, FAKE),        # cache not whole rows
    (FAKE, FAKE, 1 << 31, FAKE, 4, FAKE),     # cache past 32-bit offsets
    (None, FAKE, 1 << 20, FAKE, 4, FAKE),
    (FAKE, MISALIGNED, 1 << 20, FAKE, 4, FAKE),
    (FAKE, FAKE, 1 << 20, None, 4, FAKE),
])
def test_gather_refusals(P, args):
    assert P.csa_ceiling_gather(*args, None) == -1


def test_visible_key_pages_cover_the_scored_rows():
    from sparse_attention_decode_csa_amd import inputs as I
    sh = I.CONFIGS[3].shape.replace(batch=3, n_cap=1024, topk=64, max_len=4000)
    sp = [3999, 1000, 200]           # visible rows 1000, 250, 50 (the last fits Top-K)
    vis, scored = BC.visible_key_pages(sh, sp, 64)
    per_req = 1024 // 64
    want = list(range(0, 16)) + [per_req + i for i in range(4)]   # ceil(1000/64), ceil(250/64)
    want += [want[-1]] * (-len(want) % 8)
    assert vis.tolist() == want
    assert scored == 1000 + 250
    assert vis.size % (BC.DMA_WG_BYTES // BC.DMA_PAGE_BYTES) == 0
    with pytest.raises(ValueError):
        BC.visible_key_pages(sh, [10, 10, 10], 64)   # nothing scored
