"""The ceiling probes read what they claim to read (GPU).

A probe XORs what it loads and writes its sink only when a lane's XOR equals
a fixed constant.  With the constant planted in one dword of an otherwise
zero buffer, the sink is written exactly when the probe loads that dword, so
planting it at chosen places checks which bytes a probe covers."""
import numpy as np
import pytest
import torch

import bench_ceilings as BC

pytestmark = pytest.mark.gpu

MAGIC = 0x5A17C0DE


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available()
    return BC.load_ceilings()


def _stream_ptr():
    return torch.cuda.current_stream().cuda_stream


def _planted(nbytes, at):
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    if at is not None:
        buf[at // 4] = np.int32(np.uint32(MAGIC).view(np.int32))
    return buf


def _sink():
    return torch.zeros(16, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("at", [None, 0, 4, 131072 - 16, 131072 + 5000, 3 * 131072 + 131068])
def test_stream_dma_covers_every_byte(P, paged, at):
    nbytes = 4 * 131072
    buf, sink = _planted(nbytes, at), _sink()
    order = None
    if paged:
        n_pages = nbytes // BC.DMA_PAGE_BYTES
        order = torch.from_numpy(np.random.default_rng(3).permutation(n_pages).astype(np.int32)).cuda()
    rc = P.csa_ceiling_stream_dma(buf.data_ptr(), nbytes, None if order is None else order.data_ptr(),
                                  0 if order is None else order.numel(), sink.data_ptr(), _stream_ptr())
    assert rc == 0
    torch.cuda.synchronize()
    assert (int(sink[0].item()) != 0) == (at is not None), (paged, at)


@pytest.mark.parametrize("threads", [256, 1024])
@pytest.mark.parametrize("at", [None, 0, 65536 - 4, 65536, 5 * 65536 + 12340])
def test_stream_vec_covers_every_byte(P, at, threads):
    nbytes = 8 * 65536
    buf, sink = _planted(nbytes, at), _sink()
    assert P.csa_ceiling_stream_vec(buf.data_ptr(), nbytes, 65536, threads, sink.data_ptr(), _stream_ptr()) == 0
    torch.cuda.synchronize()
    assert (int(sink[0].item()) != 0) == (at is not None), at


@pytest.mark.parametrize("row,listed", [(5, True), (6, False), (999, True), (1023, True)])
@pytest.mark.parametrize("which", ["k", "v"])
def test_gather_reads_listed_rows_only(P, row, listed, which):
    n_rows_cache = 1024
    nbytes = n_rows_cache * BC.ROW_BYTES
    at = row * BC.ROW_BYTES + 16 * 7 + 8   # piece 7, dword 2 of the row
    k = _planted(nbytes, at if which == "k" else None)
    v = _planted(nbytes, at if which == "v" else None)
    rows = [3, 999, 5, 1023, -1, 1024, 2 ** 30, 17, 0]   # padding and out-of-range entries read zeros
    if not listed:
        rows = [r for r in rows if r != row]
    d_rows = torch.tensor(rows, dtype=torch.int32, device="cuda")
    sink = _sink()
    assert P.csa_ceiling_gather(k.data_ptr(), v.data_ptr(), nbytes, d_rows.data_ptr(), len(rows),
                                sink.data_ptr(), _stream_ptr()) == 0
    torch.cuda.synchronize()
    assert (int(sink[0].item()) != 0) == listed
