"""Host-side models of kernel index arithmetic (no GPU).

The GEMM-shaped prefill score kernel moves key rows into an LDS ring with
raw buffer loads.  The hardware range-checks only the per-lane byte offset of
such a load (the scalar offset is added unchecked), so the whole offset, key
step included, must be the per-lane one; then every access at or past the
request's n_cap rows reads zero instead of memory.  These tests replay the
kernel's offset and LDS-slot formulas on the host for every lane, wave and
issued step, including the steps the prologue issues past the last one.
"""
import itertools

import numpy as np
import pytest

GEMM_WAVES, GEMM_KEYS, STEP_KEYS, BUFS = 4, 1024, 32, 8


def tile_geometry(row_bytes):
    npr = row_bytes // 16             # 16-byte pieces per key row
    rpi = 1024 // row_bytes           # rows per 1 KiB DMA instruction
    npt = 16 * row_bytes // 1024      # DMA instructions per 16-row tile
    return npr, rpi, npt, 16 * row_bytes


def step_dma(row_bytes):
    """Per (wave, d, lane): (tile row lrow, piece, per-lane offset within the
    step, LDS byte address within the step buffer), as the kernel forms them."""
    npr, rpi, npt, tile_bytes = tile_geometry(row_bytes)
    dpw = 2 * npt // GEMM_WAVES
    out = []
    for wave, d, lane in itertools.product(range(GEMM_WAVES), range(dpw), range(64)):
        i = wave * dpw + d
        u, k = i // npt, i % npt
        r = k * rpi + lane // npr
        piece = (lane % npr) ^ (r % npr)
        lrow = u * 16 + r
        loff = lrow * row_bytes + 16 * piece
        lds = u * tile_bytes + 1024 * k + 16 * lane
        out.append((lrow, piece, loff, lds))
    return out


@pytest.mark.parametrize("row_bytes", [128, 256])   # 128-dim FP8 codes / 64-dim bf16, 128-dim bf16
def test_step_covers_every_piece_once_in_swizzled_slots(row_bytes):
    npr, _, _, tile_bytes = tile_geometry(row_bytes)
    dma = step_dma(row_bytes)
    pieces = {(lrow, piece) for (lrow, piece, _, _) in dma}
    assert len(dma) == len(pieces) == STEP_KEYS * npr     # each piece of the step's 32 rows once
    assert len({lds for *_, lds in dma}) == len(dma)       # each LDS slot written once
    for (lrow, piece, _, lds) in dma:
        u, r = lrow // 16, lrow % 16
        # the operand read of piece P of row r looks in slot P ^ (r % npr)
        assert lds == u * tile_bytes + r * row_bytes + 16 * (piece ^ (r % npr))


@pytest.mark.parametrize("row_bytes", [128, 256])
@pytest.mark.parametrize("n_cap,nmax", [(1006, 1006), (8012, 8012), (8192, 7200), (2048, 1025),
                                        (33, 33), (4096, 4096)])
def test_dma_offsets_range_checked(row_bytes, n_cap, nmax):
    """Every byte the DMA may fetch lies in rows below n_cap; everything else
    has a per-lane offset at or past the range (read as zero)."""
    dma = step_dma(row_bytes)
    rng = n_cap * row_bytes
    for key0 in range(0, nmax, GEMM_KEYS):
        nsteps = min(GEMM_KEYS // STEP_KEYS, -(-(nmax - key0) // STEP_KEYS))
        # prologue: BUFS - 1 steps whatever nsteps is; the loop issues step st + BUFS - 1
        # only while it is below nsteps
        issued = set(range(BUFS - 1)) | set(range(nsteps))
        for st in issued:
            step0 = key0 + st * STEP_KEYS
            for (lrow, piece, loff, _) in dma:
                voff = loff + step0 * row_bytes
                assert voff < 2 ** 32
                row = step0 + lrow
                if voff < rng:
                    assert row < n_cap and voff + 16 <= rng
                else:
                    assert row >= n_cap
        # every visible row of the block is fetched by some issued step
        fetched = {key0 + st * STEP_KEYS + r for st in range(nsteps) for r in range(STEP_KEYS)}
        assert set(range(key0, min(nmax, key0 + GEMM_KEYS))) <= fetched
