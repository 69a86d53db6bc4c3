"""Helpers shared by the parity tests: tolerances and comparisons.

The expected values always come from the CPU oracle (or from the pages'
mathematics); GPU results are only ever compared, never fed to the oracle.
"""
from __future__ import annotations

import json
import os
import warnings

import numpy as np

from sparse_attention_decode_csa_amd import inputs as I


class ParityRecord(UserWarning):
    """Figures of a passing parity test (boundary-exemption counts and the
    like), shown in pytest's warnings summary even in a quiet run."""


def record(test: str, **data):
    """Report one test's figures: as a ParityRecord warning, and appended as
    one JSON line to the file named by CSA_PARITY_RECORD when that is set."""
    line = json.dumps(dict(test=test, **data), default=int)
    warnings.warn(line, ParityRecord, stacklevel=2)
    path = os.environ.get("CSA_PARITY_RECORD")
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "a") as f:
            f.write(line + "\n")

# max-abs tolerance for bf16 outputs with fp32 accumulation
BF16_ATOL = 2e-2
# fp32 configuration: per (token, head) row, max |gpu - ref| <= 1e-5 * max |ref|
F32_ROW_RTOL = 1e-5
U32 = 2.0 ** -24


def score_error_bound(shape, inp, tok_rows):
    """Bound on |gpu score - exact score| for every (b, s, j) scored.

    The dot of each head is a sum of Di exactly representable products (bf16)
    or rounded fp32 products; then relu, one product with w and Hi-1 additions
    in fp32, plus the oracle's own final rounding.  With u = 2^-24 the error of
    any summation order is at most (Di + Hi + 3) u sum_h w_h sum_c |q_hc k_jc|.
    With an FP8 key cache (inp holds k_idx8 / k_scale) the keys are the
    dequantised values, and the per-row scale applied to the head sum is one
    more rounding: (Di + Hi + 4).
    Since w >= 0, sum_h w_h sum_c |q_hc k_jc| = sum_c |k_jc| (sum_h w_h |q_hc|):
    one matrix-vector product per token, key magnitudes formed once per request.
    """
    dt = shape.dtype
    q = np.abs(I.as_float(inp["q_idx"], dt).astype(np.float64))
    w = inp["w"].astype(np.float64)
    fp8 = "k_idx8" in inp
    terms = shape.idx_dim + shape.idx_heads + (4 if fp8 else 3)
    bound = {}
    kabs_b, kabs = None, None
    for (b, s, n) in tok_rows:
        if b != kabs_b:
            nmax = max(nn for (bb, _, nn) in tok_rows if bb == b)
            if fp8:
                kabs = np.abs(e4m3_values(inp["k_idx8"][b, :nmax])) * \
                    inp["k_scale"][b, :nmax, None].astype(np.float64)
            else:
                kabs = np.abs(I.as_float(inp["k_idx"][b, :nmax], dt).astype(np.float64))
            kabs_b = b
        v = w[b, s] @ q[b, s]          # sum_h w_h |q_hc|
        bound[(b, s)] = terms * U32 * (kabs[:n] @ v)
    return bound


_E4M3 = None


def e4m3_values(codes):
    """E4M3 code -> value through the oracle's (pinned) decoder."""
    global _E4M3
    if _E4M3 is None:
        import oracle
        _E4M3 = np.array([oracle.e4m3_value(c) for c in range(256)])
    return _E4M3[np.asarray(codes, np.uint8)]


def token_rows(shape, start_pos):
    """(b, s, n_vis) of every token that is scored (does not fit Top-K)."""
    out = []
    for b in range(shape.batch):
        for s in range(shape.q_per_req):
            p = int(start_pos[b]) + s
            n = min((p + 1) // shape.ratio, shape.n_cap)
            if n > shape.topk:
                out.append((b, s, n))
    return out


def compare_outputs(shape, got: np.ndarray, ref: np.ndarray, tokens=None):
    """Assert the attention output matches to the stated tolerance.

    got/ref: [G, B*S, (H/G)*D] float arrays.  `tokens` restricts the check to
    a subset of flat token indices.
    """
    G, H, D = shape.out_groups, shape.heads, shape.head_dim
    T = shape.batch * shape.q_per_req
    g4 = got.reshape(G, T, H // G, D)
    r4 = ref.reshape(G, T, H // G, D)
    if tokens is not None:
        g4, r4 = g4[:, tokens], r4[:, tokens]
    assert np.isfinite(g4).all(), "non-finite GPU output"
    err = np.abs(g4.astype(np.float64) - r4.astype(np.float64))
    if shape.dtype == I.BF16:
        worst = float(err.max(initial=0.0))
        assert worst <= BF16_ATOL, f"max abs error {worst} > {BF16_ATOL}"
        return worst
    row_err = err.max(axis=-1)
    row_mag = np.abs(r4).max(axis=-1)
    ratio = row_err / np.maximum(row_mag, 1e-30)
    worst = float(ratio.max(initial=0.0))
    assert worst <= F32_ROW_RTOL, f"row-relative error {worst} > {F32_ROW_RTOL}"
    return worst


def topk_exemptions(shape, gpu_idx, ref_idx, ref_scores, bound, start_pos, tokens=None):
    """Compare end-to-end Top-K lists; return the (b, s) tokens that differ.

    A difference is allowed only at the selection boundary: every row in the
    symmetric difference must have an oracle score within the score error
    bound (on both sides) of the oracle's K-th largest score.  `tokens`
    restricts the comparison to those (b, s) pairs.
    """
    exempt = []
    K = shape.topk
    pairs = tokens if tokens is not None else [(b, s) for b in range(shape.batch)
                                               for s in range(shape.q_per_req)]
    for (b, s) in pairs:
        gi, ri = gpu_idx[b, s], ref_idx[b, s]
        if np.array_equal(gi, ri):
            continue
        p = int(start_pos[b]) + s
        n = min((p + 1) // shape.ratio, shape.n_cap)
        assert n > K, f"bypass token {(b, s)} differs"
        assert len(set(gi.tolist())) == K and (gi >= 0).all() and (gi < n).all()
        assert np.all(np.diff(gi) > 0), "GPU list not ascending"
        sc = ref_scores[b, s, :n].astype(np.float64)
        kth = np.sort(sc)[::-1][K - 1]
        bd = bound[(b, s)]
        diff = set(gi.tolist()) ^ set(ri.tolist())
        for j in diff:
            assert abs(sc[j] - kth) <= bd[j] + bd.max(), (
                f"token {(b, s)} row {j}: score {sc[j]} far from boundary {kth}")
        exempt.append((b, s, len(diff)))
    return exempt


def selection_mask(scores, n_vis, K):
    """Boolean [T, N] mask of the exact selection of each score row: the K
    largest of its first n_vis entries, lower index first among equal values
    (rows with n_vis <= K keep all of them).  numpy's partition gives each
    row's K-th largest value; the rest is counting.  A check that holds at any
    size: it compares a list with the exact selection of the scores it was
    chosen from."""
    T, N = scores.shape
    n_vis = np.asarray(n_vis)
    col = np.arange(N)[None, :]
    valid = col < n_vis[:, None]
    sc = np.where(valid, scores, -np.inf).astype(np.float32)
    kth = -np.partition(-sc, K - 1, axis=1)[:, K - 1]                 # K-th largest per row
    gt = valid & (sc > kth[:, None])
    eq = valid & (sc == kth[:, None])
    need = K - gt.sum(axis=1)
    take_eq = eq & (np.cumsum(eq, axis=1) <= need[:, None])
    sel = gt | take_eq
    fits = n_vis <= K
    sel[fits] = valid[fits]
    return sel


def list_mask(idx, N):
    """Boolean [T, N] mask of the entries >= 0 of Top-K lists idx [T, K]."""
    T, K = idx.shape
    m = np.zeros((T, N), dtype=bool)
    r, c = np.nonzero(idx >= 0)
    m[r, idx[r, c]] = True
    return m
