"""GPU parity of the lightning indexer in its edge regimes, element by element against the
oracle at the unchanged score tolerance (tests/parity.py):

  * ReLU-dominated rows: most head dot products negative, many scores exactly 0 (rows whose
    every score is 0 must come back exactly 0);
  * H^I above 64 (96 and 128 heads): the scores, the fused prefill and the paged decode;
  * score rows over more than 16K keys, where one workgroup walks several key blocks.

Formula: I[t,s] = sum_j w[t,j] ReLU(q^I[t,j] . k^I[s]) (Keye-VL-2.0 report section 2.3.1;
xllm-io review page, section 核心公式, first formula).
"""
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_02_amd as dsa
import oracle
import workloads as W
from parity import check_scores, oracle_row_scores, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _scores(x, q0, q1, Tk):
    """GPU scores of rows q0 .. q1-1 (positions q0 ..) against keys 0 .. Tk-1."""
    sl = slice(q0, q1)
    s = dsa.index_scores(x["q_idx"][sl].contiguous(), x["q_scale"][sl].contiguous(),
                         x["w"][sl].contiguous(), x["k_idx"][:Tk].contiguous(),
                         x["k_scale"][:Tk].contiguous(), q_pos0=q0)
    torch.cuda.synchronize()
    return s


def _worst(g_rows, refs, positions):
    """Largest error in units of the tolerance over the given rows (for the log)."""
    worst = 0.0
    for g, ref, pos in zip(g_rows, refs, positions):
        ref = np.asarray(ref[:pos + 1], np.float64)
        err = np.abs(np.asarray(g[:pos + 1], np.float64) - ref)
        tol = 1e-3 * np.abs(ref) + 1e-6 * np.abs(ref).max()
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(tol > 0, err / tol, np.where(err > 0, np.inf, 0.0))
        worst = max(worst, float(r.max()))
    return worst


@pytest.mark.parametrize("HI,L,q0", [(64, 1100, 0), (64, 900, 333), (64, 131, 0),
                                     (96, 700, 0), (128, 700, 0), (128, 600, 211)])
def test_index_scores_fp8_relu_dominated(HI, L, q0):
    """Most dot products negative, half the scores exactly 0, and the first 40 rows all 0."""
    _say("index fp8 ReLU-dominated", HI, L, q0)
    x = W.relu_dominated_indexer_inputs(L, HI, seed=HI * 7 + L + q0, device=DEV)
    g = to_np(_scores(x, q0, L, L))
    ref = oracle.index_scores(to_np(x["q_idx"][q0:]), to_np(x["q_scale"][q0:]), to_np(x["w"][q0:]),
                              to_np(x["k_idx"]), to_np(x["k_scale"]), oracle.FP8_E4M3, q_pos0=q0)
    pos = [q0 + i for i in range(L - q0)]
    _say("  worst error / tolerance %.3g, exact-zero scores %.2f" % (
        _worst(g, ref, pos), np.mean([np.mean(ref[i][:p + 1] == 0) for i, p in enumerate(pos)])))
    for i in range(L - q0):
        p = q0 + i
        if p < 40:         # every score of these rows is exactly 0
            assert np.all(g[i, :p + 1] == 0), "row %d: scores of an all-zero row" % p
        check_scores(g[i, :L], ref[i], p, "row %d" % p)


@pytest.mark.parametrize("HI", [96, 128])
@pytest.mark.parametrize("L,q0", [(1100, 0), (777, 523)])
def test_index_scores_fp8_many_heads(HI, L, q0):
    _say("index fp8 H^I", HI, L, q0)
    cfg = W.scaled(W.PREFILL_32K, L=L, HI=HI, seed=L + HI)
    x = W.prefill_inputs(cfg, DEV)
    g = to_np(_scores(x, q0, L, L))
    ref = oracle.index_scores(to_np(x["q_idx"][q0:]), to_np(x["q_scale"][q0:]), to_np(x["w"][q0:]),
                              to_np(x["k_idx"]), to_np(x["k_scale"]), oracle.FP8_E4M3, q_pos0=q0)
    for i in range(L - q0):
        check_scores(g[i, :L], ref[i], q0 + i, "row %d" % (q0 + i))


@pytest.mark.parametrize("HI", [96, 128])
def test_prefill_many_heads_vs_oracle(HI):
    """The fused prefill at H^I > 64 (full score rows, chunked) against the oracle."""
    from test_gpu_parity import _check_rows_vs_oracle
    cfg = W.scaled(W.PREFILL_32K, L=3000, HI=HI, k=256, chunk=1024, seed=90 + HI)
    x = W.prefill_inputs(cfg, DEV)
    out, idx = dsa.prefill(x["q"], x["k"], x["v"], x["q_idx"], x["q_scale"], x["w"], x["k_idx"],
                           x["k_scale"], cfg.k, cfg.sm_scale, chunk_rows=cfg.chunk, return_idx=True)
    torch.cuda.synchronize()
    rows = [0, 1, 254, 255, 256, 1023, 1024, 1500, 2047, 2048, 2998, 2999]
    _check_rows_vs_oracle(cfg, x, out, idx, rows, "prefill H^I=%d" % HI, "bf16")


@pytest.mark.parametrize("HI", [96, 128])
def test_decode_many_heads_vs_oracle(HI):
    """Paged decode at H^I > 64 against the oracle, every sequence."""
    from test_gpu_parity import _decode_and_check
    cfg = W.scaled(W.DECODE_PAGED, B=6, Lmin=1, Lmax=9000, k=512, HI=HI, seed=70 + HI)
    x = W.decode_inputs(cfg, DEV, lens=torch.tensor([1, 511, 513, 4097, 8193, 9000]))
    _decode_and_check(cfg, x, list(range(cfg.B)), "decode H^I=%d" % HI)


def _check_sampled_rows(x, q0, g_rows, rows, Tk, what):
    """Elementwise check of sampled rows (indices relative to q0; g_rows[i] is row rows[i]
    of a score call)."""
    qi, qs, w = (to_np(x[n][q0:q0 + max(rows) + 1]) for n in ("q_idx", "q_scale", "w"))
    refs = oracle_row_scores(qi, qs, w, to_np(x["k_idx"][:Tk]), to_np(x["k_scale"][:Tk]),
                             oracle.FP8_E4M3, rows, q_pos0=q0)
    for r, g, ref in zip(rows, g_rows, refs):
        check_scores(g[:Tk], ref, q0 + r, "%s row %d" % (what, q0 + r))
    _say("  %s: %d rows ok, worst error / tolerance %.3g" % (
        what, len(rows), _worst(g_rows, refs, [q0 + r for r in rows])))


def test_index_scores_fp8_24k_keys_sampled():
    """1000 rows against 24000 keys: three key blocks per workgroup, ragged last block."""
    _say("index fp8 24K keys")
    cfg = W.scaled(W.PREFILL_32K, L=24000, seed=2400)
    x = W.prefill_inputs(cfg, DEV)
    q0 = 23000
    g = to_np(_scores(x, q0, cfg.L, cfg.L))
    rows = [0, 1, 15, 16, 500, 983, 984, 998, 999]
    _check_sampled_rows(x, q0, g[rows], rows, cfg.L, "24K keys")


def test_index_scores_fp8_128k_last_chunk_sampled():
    """The last 8K-row chunk of the 128K clustered workload against all 131072 keys, as the
    benchmark's staged leg launches it (16 key blocks per workgroup)."""
    cfg = W.PREFILL_128K
    _say("index fp8 128K last chunk")
    x = W.prefill_inputs(cfg, DEV)
    for n in ("q", "k", "v"):
        del x[n]
    q0 = cfg.L - cfg.chunk
    s = _scores(x, q0, cfg.L, cfg.L)
    rows = [0, 1, 2047, 4096, 6000, 8176, 8190, 8191]
    g = to_np(s[rows])
    del s
    torch.cuda.empty_cache()
    _check_sampled_rows(x, q0, g, rows, cfg.L, "128K last chunk")
