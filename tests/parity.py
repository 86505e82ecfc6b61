"""Comparators between libdsa (GPU) results and the CPU oracle.

Tolerances (all written here, used by every parity test):
  * indexer scores: |I_gpu - I_ref| <= 1e-3 M + 1e-6 max_s M[t, :] with
    M = |I_ref| for w >= 0 (every workload): the plain 1e-3 relative bound on
    fp32 accumulation of the dequantised FP8 products.  A stress test with
    signed w and few heads, where cancellation makes |I_ref| meaningless as a
    scale, passes M = sum_j |w[t,j]| sum_i |q^I[t,j,i] k^I[s,i]|, the scale of
    the rounding error of the accumulated products;
  * Top-k: with tau = the oracle's k-th score of the row and
    delta = 1e-3 |tau| + 1e-6 max_s |I_ref[t, :]|, the GPU set must hold every
    s with I_ref > tau + delta and no s with I_ref < tau - delta, have exactly
    min(k, t+1) members in [0, t], ascending, then -1 padding.  When both
    sides rank the SAME fp32 scores the sets must be identical;
  * attention, always on the GPU's own Omega: |out_gpu - out_ref| <= 2e-2 for
    bf16 I/O and <= 1e-4 for fp32 I/O.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

SCORE_RTOL = 1e-3
SCORE_FLOOR = 1e-6
ATTN_TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_np(t):
    """CPU numpy copy of a torch tensor (bf16 as uint16 bits, fp8 as uint8 codes)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.uint16)
    elif t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return t.numpy()


def sample_rows(L, k, chunk=0, n_random=4, seed=0, n_edge=2):
    """Stratified sample of query rows: first and last rows, rows around k,
    chunk boundaries +-1 and seeded random rows."""
    rows = set(range(min(n_edge, L)))
    rows |= set(range(max(0, L - n_edge), L))
    for r in (k - 2, k - 1, k, k + 1):
        if 0 <= r < L:
            rows.add(r)
    if chunk and chunk < L:
        for c in range(chunk, L, chunk):
            for r in (c - 1, c):
                rows.add(r)
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, L, n_random))
    return sorted(rows)


def oracle_row_scores(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, rows, q_pos0=0, workers=16):
    """Oracle scores of the given query rows over their causal prefix: list of
    float64 arrays, row r of length q_pos0 + r + 1.  Host numpy inputs."""
    def one(r):
        pos = q_pos0 + r
        qs = None if q_scale is None else q_scale[r:r + 1]
        ks = None if k_scale is None else k_scale[:pos + 1]
        return oracle.index_scores(q_idx[r:r + 1], qs, w[r:r + 1], k_idx[:pos + 1], ks, idx_dtype,
                                   q_pos0=pos)[0]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(one, rows))


def check_scores(gpu_row, ref_row, pos, what="", mag_row=None):
    """gpu_row: fp32 scores of one row (>= pos+1 long), ref_row: float64 oracle row;
    mag_row: the error scale M of each entry (defaults to |ref_row|)."""
    ref = np.asarray(ref_row[:pos + 1], np.float64)
    got = np.asarray(gpu_row[:pos + 1], np.float64)
    mag = np.abs(ref) if mag_row is None else np.asarray(mag_row[:pos + 1], np.float64)
    floor = SCORE_FLOOR * np.max(mag)
    err = np.abs(got - ref)
    bad = err > SCORE_RTOL * mag + floor
    assert not bad.any(), "%s: %d score mismatches, worst at s=%d gpu=%r ref=%r" % (
        what, bad.sum(), int(np.argmax(err)), got[np.argmax(err)], ref[np.argmax(err)])
    tail = np.asarray(gpu_row[pos + 1:])
    assert np.all(np.isneginf(tail)), "%s: masked entries are not -inf" % what


def check_band(gpu_idx_row, ref_row, pos, k, what=""):
    """GPU index set of one row against the oracle's scores with the tolerance band."""
    ref = np.asarray(ref_row[:pos + 1], np.float64)
    n = min(k, pos + 1)
    sel = np.asarray(gpu_idx_row)
    chosen = sel[:n]
    assert np.all(sel[n:] == -1), "%s: padding is not -1" % what
    assert np.all(chosen >= 0) and np.all(chosen <= pos), "%s: index out of [0, pos]" % what
    assert np.all(np.diff(chosen) > 0), "%s: not strictly ascending" % what
    order = np.lexsort((np.arange(pos + 1), -ref))
    tau = ref[order[n - 1]]
    delta = SCORE_RTOL * abs(tau) + SCORE_FLOOR * np.max(np.abs(ref))
    must = np.nonzero(ref > tau + delta)[0]
    never = np.nonzero(ref < tau - delta)[0]
    cs = set(chosen.tolist())
    missing = [s for s in must if s not in cs]
    extra = [s for s in never if s in cs]
    assert not missing and not extra, "%s: band violation, missing %s extra %s (tau=%r)" % (
        what, missing[:5], extra[:5], tau)
    return len(cs - set(order[:n].tolist()))           # members that differ from the oracle's


def check_attn(gpu_rows, ref_rows, dtype, what=""):
    got = np.asarray(gpu_rows, np.float64)
    ref = np.asarray(ref_rows, np.float64)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = np.abs(got - ref)
    tol = ATTN_TOL[dtype]
    assert err.max() <= tol, "%s: attention max error %.3e > %.1e" % (what, err.max(), tol)
    return float(err.max())


def bf16_to_f64(a):
    """uint16 bf16 bits -> float64 (for comparing GPU outputs)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)
