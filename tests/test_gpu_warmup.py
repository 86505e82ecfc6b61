"""GPU parity of the dense warm-up stage (libdsa through its C ABI against the CPU oracle):
the warm-up indexer loss with its gradient over the scores, and the dense indexer backward.

Small cases run several 16-row and 8-row workgroups, several 256-key blocks and row ranges,
ragged tails and query chunks (q_pos0 > 0) in full; the 32K layer runs the whole step and is
checked on sampled rows and on an identity over all rows.
"""
import sys

import numpy as np
import pytest
import torch

import long_context_sparse_02_amd as dsa
import oracle
import workloads as W
from parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(L, Hq, G, seed, HI=64):
    cfg = W.scaled(W.PREFILL_32K, L=L, Hq=Hq, G=G, HI=HI, seed=seed, keys="clustered")
    return cfg, W.prefill_inputs(cfg, DEV)


def _causal_lists(Tq, Tk, q_pos0):
    s = np.arange(Tk, dtype=np.int32)[None, :]
    pos = q_pos0 + np.arange(Tq)[:, None]
    return np.where(s <= pos, s, -1).astype(np.int32)


# Tolerances.  The kernel forms each score q.K in fp32 from exact bf16 products, and p, the
# softmax of I and the KL terms in fp32 (exp2 / log2 within 2 ulp): a probability is off by a
# few 1e-7 relative, and log softmax(I) by |I| 2^-24 absolute.  dI = G softmax(I) - sum_g p
# is checked against 2e-4 of its largest magnitude, the KL of a row against 1e-4 relative
# plus G 2^-24 max |I| (the rounding of log softmax(I) weighted by sum_g sum_s p = G).
# Where the GPU's loss runs on its own fp32 scores (I_err: their difference from the oracle's
# scores), a row whose scores move by at most e moves log softmax(I) by at most 2e: the KL by
# 2 G e and dI[s] by G softmax(I)_s (exp(2e) - 1), added to the bounds.
def _check_kl(kl, dI, rkl, rdI, I, G, what, I_err=None):
    kl = np.asarray(kl, dtype=np.float64)
    err_kl = np.abs(kl - rkl)
    fin = np.isfinite(I)
    imax = np.abs(I[fin]).max()
    bound_kl = 1e-4 * np.abs(rkl) + G * imax * 2.0 ** -24 * 8 + 1e-6
    bound_dI = np.full(rdI.shape, 2e-4 * np.abs(rdI).max() + 1e-9)
    if I_err is not None:
        e = np.where(fin, np.abs(I_err), 0.0).max(axis=1)                 # per row
        bound_kl = bound_kl + 2 * G * e
        m = np.where(fin, I, -np.inf).max(axis=1, keepdims=True)
        qI = np.where(fin, np.exp(I - m), 0.0)
        qI /= qI.sum(axis=1, keepdims=True)
        bound_dI = bound_dI + G * qI * np.expm1(2 * e)[:, None] * 1.01
        _say("  %s: scores differ from the oracle's by up to %.3e" % (what, e.max()))
    _say("  %s: kl max err %.3e (max kl %.3e), bound ratio %.3f"
         % (what, err_kl.max(), np.abs(rkl).max(), (err_kl / bound_kl).max()))
    assert np.all(err_kl <= bound_kl), what
    err_dI = np.abs(np.asarray(dI, dtype=np.float64) - rdI)
    _say("  %s: dI max err %.3e (max |dI| %.3e), bound ratio %.3f"
         % (what, err_dI.max(), np.abs(rdI).max(), (err_dI / bound_dI).max()))
    assert np.all(err_dI <= bound_dI), what


@pytest.mark.parametrize("L,q_pos0,Hq,G,with_lse", [
    (300, 0, 32, 4, False), (700, 411, 32, 4, False), (400, 150, 32, 4, True),
    (333, 0, 8, 2, False), (260, 37, 16, 1, False), (200, 0, 4, 4, False),
    (250, 90, 8, 4, False), (230, 0, 32, 8, True), (150, 20, 4, 1, False),
    (170, 0, 4, 2, False), (130, 0, 1, 1, False), (140, 33, 2, 2, True)])
def test_warmup_kl_vs_oracle(L, q_pos0, Hq, G, with_lse):
    _say("warm-up kl L=%d q_pos0=%d Hq=%d G=%d lse=%s" % (L, q_pos0, Hq, G, with_lse))
    cfg, x = _case(L, Hq, G, seed=L + Hq + G)
    Tq, sl, sm = L - q_pos0, slice(q_pos0, L), cfg.sm_scale
    I = oracle.index_scores(to_np(x["q_idx"][sl]), to_np(x["q_scale"][sl]), to_np(x["w"][sl]),
                            to_np(x["k_idx"]), to_np(x["k_scale"]), oracle.FP8_E4M3, q_pos0=q_pos0)
    I32 = I.astype(np.float32)                       # the shared input, -inf beyond the prefix
    ld = (L + 3) // 4 * 4 + 4
    scores = np.full((Tq, ld), -np.inf, dtype=np.float32)
    scores[:, :L] = I32
    q_np, k_np = to_np(x["q"][sl]), to_np(x["k"])
    lse_dev = None
    if with_lse:                                     # the dense attention's own log-sum-exp
        _, lse = oracle.attn_lse(q_np, k_np, k_np, oracle.BF16, _causal_lists(Tq, L, q_pos0), G, sm)
        lse_dev = torch.from_numpy(lse.astype(np.float32)).to(DEV)
    sc = torch.from_numpy(scores).to(DEV)
    kl = dsa.indexer_warmup_kl(x["q"][sl].contiguous(), x["k"], G, sm, sc, L, q_pos0=q_pos0,
                               lse=lse_dev)
    torch.cuda.synchronize()
    rkl, rdI = oracle.indexer_warmup_kl(q_np, k_np, oracle.BF16, G, sm, I32.astype(np.float64),
                                        q_pos0=q_pos0)
    got = to_np(sc)
    causal = _causal_lists(Tq, L, q_pos0) >= 0
    assert np.all(got[:, :L][~causal] == -np.inf) and np.all(got[:, L:] == -np.inf)  # untouched
    _check_kl(to_np(kl), np.where(causal, got[:, :L], 0.0), rkl, rdI, I32, G, "L=%d" % L)
    # a divergence is never negative, up to the rounding of log softmax(I) (row 0: exactly 0)
    assert np.all(to_np(kl) >= -(G * np.abs(I32[causal]).max() * 2.0 ** -24 * 8 + 1e-6))


@pytest.mark.parametrize("q_pos0,Hq,G", [(0, 32, 4), (90, 8, 2), (37, 16, 1)])
def test_warmup_kl_scores_far_above_key0(q_pos0, Hq, G):
    """Rows whose scores at a few keys exceed their score at key 0 by ~100 (natural units,
    sm_scale q.K): the kernel's per-(row, head) sums referenced to key 0's score overflow
    there and it takes its running-maximum walk instead; the loss and dI still match the
    oracle.  Other rows (ordinary scores) share the workgroups."""
    L = 260
    _say("warm-up kl, large scores, q_pos0=%d Hq=%d G=%d" % (q_pos0, Hq, G))
    cfg, x = _case(L, Hq, G, seed=77 + Hq)
    Tq, sl, sm = L - q_pos0, slice(q_pos0, L), cfg.sm_scale
    rng = np.random.default_rng(5 + G)
    hpg = Hq // G
    q = x["q"][sl].float().cpu().numpy()
    k = x["k"].float().cpu().numpy()
    hot_keys = [20, 131, 200]
    for g in range(G):
        u = rng.choice([-3.0, 3.0], size=128)
        for s in hot_keys:
            k[s, g] = u                                          # q.K = 9 * 128 per hot pair
        for t in range(Tq):
            if (q_pos0 + t) % 3 != 1 and q_pos0 + t >= hot_keys[0]:
                q[t, g * hpg:(g + 1) * hpg] = u
    q_d = torch.from_numpy(q).bfloat16().to(DEV)
    k_d = torch.from_numpy(k).bfloat16().to(DEV)
    I = oracle.index_scores(to_np(x["q_idx"][sl]), to_np(x["q_scale"][sl]), to_np(x["w"][sl]),
                            to_np(x["k_idx"]), to_np(x["k_scale"]), oracle.FP8_E4M3, q_pos0=q_pos0)
    I32 = I.astype(np.float32)
    ld = L + 4
    scores = np.full((Tq, ld), -np.inf, dtype=np.float32)
    scores[:, :L] = I32
    sc = torch.from_numpy(scores).to(DEV)
    kl = dsa.indexer_warmup_kl(q_d, k_d, G, sm, sc, L, q_pos0=q_pos0)
    torch.cuda.synchronize()
    rkl, rdI = oracle.indexer_warmup_kl(to_np(q_d), to_np(k_d), oracle.BF16, G, sm,
                                        I32.astype(np.float64), q_pos0=q_pos0)
    causal = _causal_lists(Tq, L, q_pos0) >= 0
    got = to_np(sc)
    _check_kl(to_np(kl), np.where(causal, got[:, :L], 0.0), rkl, rdI, I32, G, "large scores")
    # the hot rows put nearly all of p on the hot keys they see
    t = Tq - 1 if (L - 1) % 3 != 1 else Tq - 2
    assert rdI[t, hot_keys].sum() < -0.9 * G


def _int_indexer(rng, T, Tk, HI):
    """FP8 codes of the integers -4..4 (every dot product exact in fp32, so both sides take
    the same ReLU decisions), positive scales, signed weights."""
    lut = np.array([0x00, 0x38, 0x40, 0x44, 0x48], dtype=np.uint8)

    def codes(shape):
        mag = rng.integers(0, 5, shape)
        c = lut[mag] | (rng.integers(0, 2, shape).astype(np.uint8) << 7)
        c[mag == 0] = 0
        return c
    return (codes((T, HI, 128)), rng.uniform(0.5, 2.0, T).astype(np.float32),
            rng.normal(size=(T, HI)).astype(np.float32), codes((Tk, 128)),
            rng.uniform(0.5, 2.0, Tk).astype(np.float32))


def _dev(*arrays):
    return [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


def _grad_bounds(qc, qs, w, kc, ks, g_bound, q_pos0=0):
    """Elementwise bounds on the dense backward's errors for per-entry errors g_bound of the
    gradient that enters it: the oracle's backward of g_bound with |w| and sign-cleared codes
    (every |q^I . k^I| term counted), i.e. sum_s g_bound |w| |k^I[s]| for dq^I,
    sum_s g_bound |x| for dw and sum_{t,j} g_bound |w| |q^I[t,j]| for dk^I."""
    return oracle.index_scores_bwd_dense(qc & 0x7F, qs, np.abs(w), kc & 0x7F, ks, oracle.FP8_E4M3,
                                         g_bound, q_pos0=q_pos0)


def _relu_flip_bounds(qc, qs, w, kc, ks, g_abs):
    """Extra error bounds for one query row where the matrix core's fp32 sum of x = q^I . k^I
    (FP8 products spanning 2^-18 .. 2^17.6: not exact in fp32) may take the ReLU decision the
    other way: a (head, key) pair is in doubt when |x| <= 2^-17 sum_i |q_i k_i| (128 terms of
    fp32 rounding).  Such a pair can add or drop |g| |w| |k^I| in dq^I and |g| |x| in dw.
    x is exact in float64 here (at most 43 significant bits)."""
    lut = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    qv, kv = lut[qc[0]], lut[kc]                               # [HI, 128], [n, 128] code values
    x = qv @ kv.T
    a = np.abs(qv) @ np.abs(kv).T
    doubt = (np.abs(x) <= 2.0 ** -17 * a) & (a > 0)
    gk = doubt * g_abs[None, :]                                 # [HI, n]
    kdeq = np.abs(kv) * ks[:, None].astype(np.float64)
    fq = np.abs(w[0]).astype(np.float64)[:, None] * (gk @ kdeq)
    fw = (gk * np.abs(x) * float(qs[0]) * ks[None, :].astype(np.float64)).sum(axis=1)
    return fq[None], fw[None]


def _check_grads(got, ref, bounds, what):
    for name, g_, r_, b_ in zip(("dq^I", "dw", "dk^I"), got, ref, bounds):
        err = np.abs(np.asarray(g_, dtype=np.float64) - r_)
        lim = b_ * 1.01 + 1e-9 * np.abs(r_).max()
        _say("  %s %s: max err %.3e of max |ref| %.3e, bound ratio %.3f"
             % (what, name, err.max(), np.abs(r_).max(), (err / lim).max()))
        assert np.all(err <= lim), (what, name)


@pytest.mark.parametrize("T,q_pos0,HI,extra", [(200, 0, 64, 0), (150, 333, 64, 0), (97, 40, 16, 0),
                                                (120, 0, 48, 0), (300, 700, 32, 0),
                                                (100, 50, 64, 900)])
def test_index_scores_bwd_dense_vs_oracle(T, q_pos0, HI, extra):
    """dq^I, dw and dk^I against the oracle; entries of g beyond each row's prefix are NaN and
    must be ignored; two calls give identical bits; two row chunks accumulate dk^I.  With
    `extra` keys past the last row's position, whole key blocks are seen by no row: their
    dk^I must stay exactly zero."""
    _say("dense indexer bwd T=%d q_pos0=%d HI=%d extra=%d" % (T, q_pos0, HI, extra))
    rng = np.random.default_rng(T + HI + q_pos0)
    Tk = q_pos0 + T + extra
    qc, qs, w, kc, ks = _int_indexer(rng, T, Tk, HI)
    causal = _causal_lists(T, Tk, q_pos0) >= 0
    ld = Tk + 4
    g = np.full((T, ld), np.nan, dtype=np.float32)
    g[:, :Tk] = np.where(causal, rng.normal(size=(T, Tk)), np.nan)
    a = _dev(qc, qs, w, kc, ks, g)
    dq, dw, dk = dsa.index_scores_bwd_dense(*a, Tk, q_pos0=q_pos0)
    dq2, dw2, dk2 = dsa.index_scores_bwd_dense(*a, Tk, q_pos0=q_pos0)
    # the same rows in two chunks, dk^I accumulated over both
    h = T // 2
    dkc = torch.zeros_like(dk)
    parts = []
    for r0, r1 in ((0, h), (h, T)):
        b = _dev(qc[r0:r1], qs[r0:r1], w[r0:r1], kc, ks, g[r0:r1])
        parts.append(dsa.index_scores_bwd_dense(*b, Tk, q_pos0=q_pos0 + r0, dk=dkc)[:2])
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dw, dw2) and torch.equal(dk, dk2)
    assert torch.equal(torch.cat([parts[0][0], parts[1][0]]), dq)     # per row: same work
    assert torch.equal(torch.cat([parts[0][1], parts[1][1]]), dw)
    assert (dkc - dk).abs().max().item() <= 1e-5 * dk.abs().max().item()
    if extra:
        assert torch.count_nonzero(dk[q_pos0 + T:]).item() == 0
    gd = np.where(causal, g[:, :Tk], 0.0).astype(np.float64)
    rq, rw, rk = oracle.index_scores_bwd_dense(qc, qs, w, kc, ks, oracle.FP8_E4M3, gd,
                                               q_pos0=q_pos0)
    # dq and dk take G = dI w [x > 0] rounded to bf16 into the matrix products (2^-8 relative
    # per term, the unit roundoff of bf16); dw is accumulated in fp32 from exact products (a
    # few 2^-24 of the same sums)
    _check_grads((to_np(dq), to_np(dw), to_np(dk)), (rq, rw, rk),
                 _grad_bounds(qc, qs, w, kc, ks, 2.0 ** -8 * np.abs(gd), q_pos0), "T=%d" % T)


def test_warmup_step_chain_vs_oracle():
    """The whole warm-up step: full-row scores, the loss with dI in place, the dense backward;
    against the oracle's chain.  Indexer codes of the integers -4..4, so both sides take the
    same ReLU decisions (real-valued codes: the full-size test below)."""
    L, Hq, G = 600, 32, 4
    _say("warm-up step chain L=%d" % L)
    cfg, x = _case(L, Hq, G, seed=4242)
    qc, qs, w, kc, ks = _int_indexer(np.random.default_rng(4242), L, L, 64)
    x["q_idx"], x["q_scale"], x["w"], x["k_idx"], x["k_scale"] = _dev(qc, qs, w, kc, ks)
    sm = cfg.sm_scale
    scores = dsa.index_scores(x["q_idx"], x["q_scale"], x["w"], x["k_idx"], x["k_scale"])
    I_gpu = scores[:, :L].clone()
    kl = dsa.indexer_warmup_kl(x["q"], x["k"], G, sm, scores, L)
    dq, dw, dk = dsa.index_scores_bwd_dense(x["q_idx"], x["q_scale"], x["w"], x["k_idx"],
                                            x["k_scale"], scores, L)
    torch.cuda.synchronize()
    ia = [to_np(x[n]) for n in ("q_idx", "q_scale", "w", "k_idx", "k_scale")]
    I = oracle.index_scores(*ia, oracle.FP8_E4M3)
    rkl, rdI = oracle.indexer_warmup_kl(to_np(x["q"]), to_np(x["k"]), oracle.BF16, G, sm, I)
    rq, rw, rk = oracle.index_scores_bwd_dense(*ia, oracle.FP8_E4M3, rdI)
    causal = _causal_lists(L, L, 0) >= 0
    dI = np.where(causal, to_np(scores)[:, :L], 0.0).astype(np.float64)
    _check_kl(to_np(kl), dI, rkl, rdI, I, G, "chain",
              I_err=np.where(causal, to_np(I_gpu), 0.0) - np.where(causal, I, 0.0))
    # the GPU's backward runs on its own dI: its difference from the oracle's dI, plus the
    # bf16 rounding of G, bounds the gradients' errors
    g_bound = np.abs(dI - rdI) + 2.0 ** -8 * np.abs(dI)
    _check_grads((to_np(dq), to_np(dw), to_np(dk)), (rq, rw, rk),
                 _grad_bounds(*ia, g_bound), "chain")


def test_warmup_step_full_size_sampled():
    """The 32K layer's warm-up step as the benchmark runs it.  Sampled rows of the loss, dI,
    dq^I and dw against the oracle (which recomputes those rows' scores itself); dk^I against
    an identity over all rows: I is homogeneous of degree 1 in k^I and in q^I, so
    sum_s dk[s] . k[s] = sum_{t,j} dq[t,j] . q[t,j] = sum_{t,j} w[t,j] dw[t,j]
    (dequantised k and q)."""
    cfg = W.PREFILL_32K
    L, G, sm = cfg.L, cfg.G, cfg.sm_scale
    _say("warm-up step", cfg.name)
    x = W.prefill_inputs(cfg, DEV)
    scores = dsa.index_scores(x["q_idx"], x["q_scale"], x["w"], x["k_idx"], x["k_scale"])
    rows = [0, 1, 15, 16, 4095, 20011, L - 1]
    r_t = torch.tensor(rows, device=DEV)
    I_gpu = to_np(scores[r_t]).astype(np.float64)
    kl = dsa.indexer_warmup_kl(x["q"], x["k"], G, sm, scores, L)
    dq, dw, dk = dsa.index_scores_bwd_dense(x["q_idx"], x["q_scale"], x["w"], x["k_idx"],
                                            x["k_scale"], scores, L)
    # the same with |dI|: sum_s |dI| ReLU(x) per head bounds the identity's rounding below
    _, dw_abs, _ = dsa.index_scores_bwd_dense(x["q_idx"], x["q_scale"], x["w"], x["k_idx"],
                                              x["k_scale"], scores.abs(), L)
    torch.cuda.synchronize()
    assert torch.isfinite(kl).all() and torch.isfinite(dk).all() and torch.isfinite(dq).all()
    ia = [to_np(x[n]) for n in ("q_idx", "q_scale", "w", "k_idx", "k_scale")]
    q_np, k_np = to_np(x["q"]), to_np(x["k"])
    kl_np, dI_np = to_np(kl), to_np(scores[r_t])
    dq_np, dw_np = to_np(dq[r_t]), to_np(dw[r_t])
    for i, t in enumerate(rows):
        n = t + 1
        I = oracle.index_scores(ia[0][t:t + 1], ia[1][t:t + 1], ia[2][t:t + 1], ia[3][:n],
                                ia[4][:n], oracle.FP8_E4M3, q_pos0=t)
        rkl, rdI = oracle.indexer_warmup_kl(q_np[t:t + 1], k_np[:n], oracle.BF16, G, sm, I, q_pos0=t)
        _check_kl(kl_np[t:t + 1], dI_np[i:i + 1, :n], rkl, rdI, I, G, "row %d" % t,
                  I_err=I_gpu[i:i + 1, :n] - I)
        row = [ia[0][t:t + 1], ia[1][t:t + 1], ia[2][t:t + 1], ia[3][:n], ia[4][:n]]
        rq, rw, _ = oracle.index_scores_bwd_dense(*row, oracle.FP8_E4M3, rdI, q_pos0=t)
        dI_t = dI_np[i:i + 1, :n].astype(np.float64)
        bq, bw, _ = _grad_bounds(*row, np.abs(dI_t - rdI) + 2.0 ** -8 * np.abs(dI_t), t)
        fq, fw = _relu_flip_bounds(*row, np.abs(dI_t[0]))
        _check_grads((dq_np[i:i + 1], dw_np[i:i + 1]), (rq, rw), (bq + fq, bw + fw), "row %d" % t)
    lut = torch.tensor([oracle.e4m3_to_double(c) for c in range(256)], dtype=torch.float64,
                       device=DEV)
    kdeq = lut[x["k_idx"].long()] * x["k_scale"].double()[:, None]
    qdeq = lut[x["q_idx"].long()] * x["q_scale"].double()[:, None, None]
    a = (dk.double() * kdeq).sum().item()
    b = (dq.double() * qdeq).sum().item()
    c = (x["w"].double() * dw.double()).sum().item()
    scale = (x["w"].double().abs() * dw_abs.double()).sum().item()
    _say("  identity: <dk,k> %.6e  <dq,q> %.6e  <w,dw> %.6e  (scale %.3e)" % (a, b, c, scale))
    assert abs(a - c) <= 1e-2 * scale and abs(b - c) <= 1e-2 * scale
