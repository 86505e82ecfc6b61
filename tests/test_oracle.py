"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: each test checks it against a
hand-computed value, a library routine, a closed form, an invariant, or a
brute-force characterisation on a tiny input.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from golden_io import indexer_hand, topk_ties
from workloads import quantize_e4m3_per_token

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


# ------------------------------------------------------------------ decoding

def test_e4m3_decode_matches_torch_all_codes():
    """Every one of the 256 OCP E4M3 codes decodes as torch's float8_e4m3fn does."""
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                      # S.1111.111 only
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_decode_special_values():
    """Values the OCP E4M3 definition fixes: max 448, subnormals, -0."""
    assert oracle.e4m3_to_double(0x7E) == 448.0
    assert oracle.e4m3_to_double(0xFE) == -448.0
    assert oracle.e4m3_to_double(0x01) == 2.0 ** -9       # smallest subnormal
    assert oracle.e4m3_to_double(0x07) == 7 * 2.0 ** -9   # largest subnormal
    assert oracle.e4m3_to_double(0x08) == 2.0 ** -6       # smallest normal
    assert oracle.e4m3_to_double(0x38) == 1.0
    assert math.copysign(1.0, oracle.e4m3_to_double(0x80)) == -1.0
    assert math.isnan(oracle.e4m3_to_double(0x7F))


def test_bf16_decode_matches_torch():
    bits = torch.tensor([0x0000, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x8000, 0x3C00],
                        dtype=torch.int32).to(torch.uint16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits.to(torch.int32)])
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------- indexer

def _hand_case():
    d = indexer_hand()
    HI, dI = d["HI"], d["dI"]
    T = len(d["k"])
    q = np.zeros((T, HI, dI), np.uint8)
    qs = np.zeros(T, np.float32)
    for (t, j), (codes, sc) in d["q"].items():
        q[t, j] = codes
        qs[t] = sc
    k = np.array([d["k"][s][0] for s in range(T)], np.uint8)
    ks = np.array([d["k"][s][1] for s in range(T)], np.float32)
    w = np.array([d["w"][t] for t in range(T)], np.float32)
    return d, q, qs, w, k, ks


def test_indexer_hand_computed_golden():
    """tests/golden/indexer_hand.txt: scores worked out by hand from the formula."""
    d, q, qs, w, k, ks = _hand_case()
    I = oracle.index_scores(q, qs, w, k, ks, oracle.FP8_E4M3)
    T = I.shape[0]
    for t in range(T):
        for s in range(T):
            if s > t:
                assert I[t, s] == -np.inf
            else:
                assert I[t, s] == d["I"][(t, s)], (t, s)


def test_hand_codes_are_the_values_the_fixture_claims():
    """The fixture's hex codes decode (by torch) to the small exact values used in the working."""
    d, q, qs, w, k, ks = _hand_case()
    vals = torch.from_numpy(k).view(torch.float8_e4m3fn).float().numpy()
    assert vals.tolist() == [[1, 0, 2, -1], [0.5, 1, -1, 0], [-2, 1, 0, 1.5]]


def test_topk_of_hand_scores_golden():
    d, q, qs, w, k, ks = _hand_case()
    I = oracle.index_scores(q, qs, w, k, ks, oracle.FP8_E4M3)
    for kk, t, expect in d["topk"]:
        idx, _ = oracle.topk(I[t:t + 1], [t], kk)
        got = [x for x in idx[0].tolist() if x >= 0]
        assert got == expect, (kk, t, got)


def _rand_fp8_case(rng, T, HI, dI, signed_w=False):
    qf = torch.from_numpy(rng.standard_normal((T, HI, dI)).astype(np.float32))
    kf = torch.from_numpy(rng.standard_normal((T, dI)).astype(np.float32))
    q, qs = quantize_e4m3_per_token(qf)
    k, ks = quantize_e4m3_per_token(kf)
    w = rng.uniform(-1 if signed_w else 0, 1, (T, HI)).astype(np.float32)
    return q.numpy(), qs.numpy(), w, k.numpy(), ks.numpy()


def test_indexer_single_head_unit_weight_is_relu_of_dot():
    """Special case H^I = 1, w = 1: I[t,s] = ReLU(q^I[t] . k^I[s]) (a plain matmul)."""
    rng = np.random.default_rng(0)
    q, qs, w, k, ks = _rand_fp8_case(rng, 12, 1, 32)
    w[:] = 1.0
    I = oracle.index_scores(q, qs, w, k, ks, oracle.FP8_E4M3)
    qv = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy()[:, 0, :] * qs[:, None]
    kv = torch.from_numpy(k).view(torch.float8_e4m3fn).double().numpy() * ks[:, None]
    ref = np.maximum(qv @ kv.T, 0.0)
    tri = np.tril(np.ones_like(ref, dtype=bool))
    assert np.allclose(I[tri], ref[tri], rtol=1e-13, atol=1e-13)
    assert np.all(I[~tri] == -np.inf)


def test_indexer_all_negative_dots_score_zero():
    """Every head's dot product negative => I = 0 whatever w is."""
    one, neg = 0x38, 0xB8
    q = np.full((2, 3, 4), one, np.uint8)
    k = np.array([[one] * 4, [neg] * 4], np.uint8)         # k1 = -q direction
    qs = np.ones(2, np.float32)
    ks = np.ones(2, np.float32)
    w = np.array([[0.3, 0.7, 5.0], [1.0, 2.0, 3.0]], np.float32)
    I = oracle.index_scores(q, qs, w, k, ks, oracle.FP8_E4M3)
    assert I[1, 1] == 0.0
    assert I[1, 0] == pytest.approx(4.0 * (1 + 2 + 3))


def test_indexer_linear_in_w_and_positive_for_positive_w():
    rng = np.random.default_rng(1)
    q, qs, w1, k, ks = _rand_fp8_case(rng, 20, 4, 16, signed_w=True)
    w2 = rng.uniform(-1, 1, w1.shape).astype(np.float32)
    I1 = oracle.index_scores(q, qs, w1, k, ks, oracle.FP8_E4M3)
    I2 = oracle.index_scores(q, qs, w2, k, ks, oracle.FP8_E4M3)
    I12 = oracle.index_scores(q, qs, (w1.astype(np.float64) + w2).astype(np.float32), k, ks,
                              oracle.FP8_E4M3)
    tri = np.isfinite(I1)
    # w1 + w2 rounds to fp32; compare against the exactly representable sums only
    exact = (w1.astype(np.float64) + w2 == (w1 + w2).astype(np.float64)).all()
    if exact:
        assert np.allclose(I12[tri], I1[tri] + I2[tri], rtol=1e-12, atol=1e-12)
    wpos = np.abs(w1)
    Ip = oracle.index_scores(q, qs, wpos, k, ks, oracle.FP8_E4M3)
    assert np.all(Ip[tri] >= 0)


def test_indexer_key_scale_law():
    """Doubling k_scale[s] doubles column s exactly (scales are positive, ReLU is homogeneous)."""
    rng = np.random.default_rng(2)
    q, qs, w, k, ks = _rand_fp8_case(rng, 16, 4, 16, signed_w=True)
    I = oracle.index_scores(q, qs, w, k, ks, oracle.FP8_E4M3)
    ks2 = ks.copy()
    ks2[5] *= 2
    I2 = oracle.index_scores(q, qs, w, k, ks2, oracle.FP8_E4M3)
    assert np.array_equal(I2[:, 5][5:], 2 * I[:, 5][5:])
    other = [s for s in range(16) if s != 5]
    assert np.array_equal(I2[:, other], I[:, other])


def test_indexer_head_permutation_invariance_and_key_locality():
    rng = np.random.default_rng(3)
    q, qs, w, k, ks = _rand_fp8_case(rng, 16, 6, 16, signed_w=True)
    I = oracle.index_scores(q, qs, w, k, ks, oracle.FP8_E4M3)
    perm = rng.permutation(6)
    Ip = oracle.index_scores(np.ascontiguousarray(q[:, perm]), qs, np.ascontiguousarray(w[:, perm]),
                             k, ks, oracle.FP8_E4M3)
    fin = np.isfinite(I)
    assert np.allclose(Ip[fin], I[fin], rtol=1e-13, atol=1e-13)
    # changing key 3 only changes column 3
    k2 = k.copy()
    k2[3] = rng.integers(0, 0x77, 16)
    I3 = oracle.index_scores(q, qs, w, k2, ks, oracle.FP8_E4M3)
    cols = [s for s in range(16) if s != 3]
    assert np.array_equal(I3[:, cols], I[:, cols])


def test_indexer_rows_subset_and_query_offset():
    """Sampled rows equal the full computation; q_pos0 shifts the causal boundary."""
    rng = np.random.default_rng(4)
    q, qs, w, k, ks = _rand_fp8_case(rng, 24, 4, 16)
    I = oracle.index_scores(q, qs, w, k, ks, oracle.FP8_E4M3)
    rows = np.array([0, 7, 23], np.int32)
    Ir = oracle.index_scores(q, qs, w, k, ks, oracle.FP8_E4M3, rows=rows)
    assert np.array_equal(Ir, I[rows])
    # the last 8 queries alone, at positions 16..23
    Io = oracle.index_scores(q[16:], qs[16:], w[16:], k, ks, oracle.FP8_E4M3, q_pos0=16)
    assert np.array_equal(Io, I[16:])


def test_indexer_f32_matches_float64_matmul_definition_on_tiny():
    """fp32 indexer: brute force over heads with numpy float64 matmuls."""
    rng = np.random.default_rng(5)
    T, HI, dI = 10, 3, 8
    q = rng.standard_normal((T, HI, dI)).astype(np.float32)
    k = rng.standard_normal((T, dI)).astype(np.float32)
    w = rng.uniform(-1, 1, (T, HI)).astype(np.float32)
    I = oracle.index_scores(q, None, w, k, None, oracle.F32)
    for t in range(T):
        for s in range(T):
            if s > t:
                assert I[t, s] == -np.inf
                continue
            dots = q[t].astype(np.float64) @ k[s].astype(np.float64)
            assert I[t, s] == pytest.approx(float(np.sum(w[t] * np.maximum(dots, 0))), rel=1e-12, abs=1e-12)


# --------------------------------------------------------------------- top-k

def test_topk_golden_ties():
    scores, cases = topk_ties()
    for kk, expect in cases:
        idx, kth = oracle.topk(np.array([scores]), [len(scores) - 1], kk)
        got = idx[0].tolist()
        assert got[:len(expect)] == expect, (kk, got)
        assert all(x == -1 for x in got[len(expect):])


def _check_topk_definition(row, pos, kk, sel):
    """The unique answer: n = min(k, pos+1) distinct positions in [0, pos], ascending, and every
    selected position beats every unselected one (higher score, or equal score and lower index)."""
    n = min(kk, pos + 1)
    chosen = [x for x in sel if x >= 0]
    assert len(chosen) == n and all(x == -1 for x in sel[n:])
    assert chosen == sorted(set(chosen))
    assert all(0 <= x <= pos for x in chosen)
    rest = [s for s in range(pos + 1) if s not in set(chosen)]
    for a in chosen:
        for b in rest:
            assert row[a] > row[b] or (row[a] == row[b] and a < b), (a, b)


def test_topk_brute_force_tiny_with_heavy_ties():
    rng = np.random.default_rng(6)
    for trial in range(200):
        L = int(rng.integers(1, 14))
        row = rng.integers(-3, 4, L).astype(np.float64) * 0.5
        row[rng.random(L) < 0.2] *= -1  # introduce -0.0 where row is 0
        pos = int(rng.integers(0, L))
        kk = int(rng.integers(1, L + 3))
        idx, kth = oracle.topk(row[None, :], [pos], kk)
        sel = idx[0].tolist()
        _check_topk_definition(row, pos, kk, sel)
        # exhaustive: among all n-subsets of [0,pos], the selected one maximises the sorted scores
        n = min(kk, pos + 1)
        if pos < 9:
            best = max(itertools.combinations(range(pos + 1), n),
                       key=lambda c: (sorted((row[i] for i in c), reverse=True), [-i for i in c]))
            assert sorted(best) == [x for x in sel if x >= 0]


def test_topk_dense_when_k_covers_prefix():
    rng = np.random.default_rng(7)
    row = rng.standard_normal(50)
    for pos in (0, 1, 10, 49):
        idx, _ = oracle.topk(row[None, :], [pos], 64)
        assert idx[0, :pos + 1].tolist() == list(range(pos + 1))
        assert np.all(idx[0, pos + 1:] == -1)


def test_topk_kth_is_the_kth_largest():
    rng = np.random.default_rng(8)
    row = rng.standard_normal(100)
    idx, kth = oracle.topk(row[None, :], [99], 10)
    assert kth[0] == np.sort(row)[::-1][9]


# ----------------------------------------------------------------- attention

def _attn_inputs(rng, T, Hq, G, d, dtype):
    q = rng.standard_normal((T, Hq, d)).astype(np.float32) / math.sqrt(d)
    k = rng.standard_normal((T, G, d)).astype(np.float32) / math.sqrt(d)
    v = rng.standard_normal((T, G, d)).astype(np.float32)
    if dtype == oracle.BF16:
        conv = lambda a: torch.from_numpy(a).to(torch.bfloat16)
        return conv(q), conv(k), conv(v)
    return q, k, v


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_attention_equals_dense_causal_sdpa_when_k_covers_prefix(dtype):
    """k >= t+1 makes DSA dense: compare with torch's causal SDPA in float64, KV heads repeated."""
    rng = np.random.default_rng(9)
    T, Hq, G, d = 40, 8, 2, 32
    q, k, v = _attn_inputs(rng, T, Hq, G, d, dtype)
    idx = np.array([[s if s <= t else -1 for s in range(T)] for t in range(T)], np.int32)
    out = oracle.sparse_gqa_attn(q, k, v, dtype, idx, Hq, G, 1 / math.sqrt(d))
    tq = torch.as_tensor(q).double().permute(1, 0, 2)
    tk = torch.as_tensor(k).double().repeat_interleave(Hq // G, dim=1).permute(1, 0, 2)
    tv = torch.as_tensor(v).double().repeat_interleave(Hq // G, dim=1).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           scale=1 / math.sqrt(d))
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(10)
    T, Hq, G, d = 16, 4, 2, 8
    q, k, v = _attn_inputs(rng, T, Hq, G, d, oracle.F32)
    sm = 0.3
    # t = 0 attends only to itself: output = V[0, g]
    idx0 = np.full((T, 4), -1, np.int32)
    idx0[0, 0] = 0
    out = oracle.sparse_gqa_attn(q, k, v, oracle.F32, idx0, Hq, G, sm, rows=[0])
    for h in range(Hq):
        assert np.allclose(out[0, h], v[0, h // 2], atol=1e-15, rtol=0)
    # identical keys => uniform weights => mean of the selected V rows
    k_same = np.repeat(k[:1], T, axis=0)
    sel = np.array([[1, 4, 9, 12]] * T, np.int32)
    out = oracle.sparse_gqa_attn(q, k_same, v, oracle.F32, sel, Hq, G, sm, rows=[13])
    for h in range(Hq):
        assert np.allclose(out[0, h], v[[1, 4, 9, 12], h // 2].astype(np.float64).mean(0), atol=1e-14)
    # identical V rows => that row, whatever the weights
    v_same = np.repeat(v[3:4], T, axis=0)
    out = oracle.sparse_gqa_attn(q, k, v_same, oracle.F32, sel, Hq, G, sm, rows=[13])
    for h in range(Hq):
        assert np.allclose(out[0, h], v_same[0, h // 2], atol=1e-14)
    # an empty set gives zeros
    out = oracle.sparse_gqa_attn(q, k, v, oracle.F32, np.full((T, 4), -1, np.int32), Hq, G, sm, rows=[5])
    assert np.all(out == 0)


def test_attention_two_keys_closed_form():
    """Two selected keys: weights are the logistic of the logit difference."""
    rng = np.random.default_rng(11)
    T, Hq, G, d = 8, 2, 1, 4
    q, k, v = _attn_inputs(rng, T, Hq, G, d, oracle.F32)
    sm = 0.7
    sel = np.full((T, 3), -1, np.int32)
    sel[6, :2] = [2, 5]
    out = oracle.sparse_gqa_attn(q, k, v, oracle.F32, sel, Hq, G, sm, rows=[6])
    for h in range(Hq):
        l2 = sm * float(np.dot(q[6, h].astype(np.float64), k[2, 0]))
        l5 = sm * float(np.dot(q[6, h].astype(np.float64), k[5, 0]))
        p2 = 1.0 / (1.0 + math.exp(l5 - l2))
        expect = p2 * v[2, 0].astype(np.float64) + (1 - p2) * v[5, 0]
        assert np.allclose(out[0, h], expect, atol=1e-14)


def test_attention_invariances():
    rng = np.random.default_rng(12)
    T, Hq, G, d = 24, 8, 4, 16
    q, k, v = _attn_inputs(rng, T, Hq, G, d, oracle.F32)
    sel = np.stack([rng.permutation(T)[:6] for _ in range(T)]).astype(np.int32)
    out = oracle.sparse_gqa_attn(q, k, v, oracle.F32, sel, Hq, G, 0.25)
    perm = np.ascontiguousarray(sel[:, ::-1])
    outp = oracle.sparse_gqa_attn(q, k, v, oracle.F32, perm, Hq, G, 0.25)
    assert np.allclose(out, outp, atol=1e-14)
    # group 0's output depends only on group 0's K/V
    k2, v2 = k.copy(), v.copy()
    k2[:, 1:] = rng.standard_normal(k2[:, 1:].shape)
    v2[:, 1:] = rng.standard_normal(v2[:, 1:].shape)
    out2 = oracle.sparse_gqa_attn(q, k2, v2, oracle.F32, sel, Hq, G, 0.25)
    assert np.array_equal(out2[:, :2], out[:, :2])
    assert not np.allclose(out2[:, 2:], out[:, 2:])
    # the same index set serves every group: head h in group h // (Hq/G)
    assert np.array_equal(out[:, 0], oracle.sparse_gqa_attn(q, k, v, oracle.F32, sel, Hq, G, 0.25)[:, 0])


# ---------------------------------------------------------------- paged decode

def _paged_from_contiguous(rng, arrays, L, bs, extra_blocks=3):
    """Scatter contiguous per-token arrays into a shuffled paged layout."""
    nb = (L + bs - 1) // bs
    NB = nb + extra_blocks
    perm = rng.permutation(NB)[:nb].astype(np.int32)
    out = []
    for a in arrays:
        paged = np.zeros((NB, bs) + a.shape[1:], a.dtype)
        for i in range(nb):
            n = min(bs, L - i * bs)
            paged[perm[i], :n] = a[i * bs:i * bs + n]
        out.append(paged)
    return perm, out


def test_decode_equals_prefill_row_through_block_table():
    """Decode of a sequence of length t+1 equals prefill row t (paged vs contiguous addressing)."""
    rng = np.random.default_rng(13)
    L, HI, dI, Hq, G, d, kk, bs = 45, 4, 16, 4, 2, 8, 7, 8
    q_idx, qs, w, k_idx, ks = _rand_fp8_case(rng, L, HI, dI)
    q = rng.standard_normal((L, Hq, d)).astype(np.float32)
    k = rng.standard_normal((L, G, d)).astype(np.float32)
    v = rng.standard_normal((L, G, d)).astype(np.float32)
    I = oracle.index_scores(q_idx, qs, w, k_idx, ks, oracle.FP8_E4M3)
    idx, kth = oracle.topk(I, np.arange(L), kk)
    out = oracle.sparse_gqa_attn(q, k, v, oracle.F32, idx, Hq, G, 0.4)
    for t in (0, 6, 7, 30, 44):
        n = t + 1
        perm, (kc, vc, kic, ksc) = _paged_from_contiguous(rng, [k[:n], v[:n], k_idx[:n], ks[:n]], n, bs)
        bt = perm[None, :]
        i2, kth2, o2 = oracle.decode(q[t:t + 1], q_idx[t:t + 1], qs[t:t + 1], w[t:t + 1], kic, ksc,
                                     kc, vc, oracle.F32, bt, np.array([n], np.int32), bs, kk, 0.4)
        assert np.array_equal(i2[0], idx[t])
        assert kth2[0] == kth[t]
        assert np.allclose(o2[0], out[t], atol=1e-13)


# ------------------------------------------------------------ FP8 quantisation

def _quant_torch(x):
    """Per-token absmax E4M3 quantisation with torch's own float8 cast (the harness recipe)."""
    return quantize_e4m3_per_token(torch.as_tensor(x))


def test_quantize_matches_torch_float8_cast():
    """The oracle's exhaustive-search rounding against torch's float8_e4m3fn conversion, on
    normal rows, heavy-tailed rows, rows of tiny values (subnormal codes) and an all-zero row."""
    g = np.random.default_rng(11)
    rows = [g.standard_normal(512), g.standard_cauchy(512), g.standard_normal(512) * 1e-6,
            np.zeros(512), np.concatenate([[448.0], g.uniform(-448, 448, 511)])]
    x = np.stack(rows).astype(np.float32)
    codes, scale = oracle.quantize_e4m3(x)
    tc, ts = _quant_torch(x)
    assert np.array_equal(scale, ts.numpy())
    assert np.array_equal(codes, tc.numpy())
    assert scale[3] == 1.0 and np.all(codes[3] == 0)


def test_quantize_rounds_ties_to_even_codes():
    """Hand-worked row with scale exactly 1 (the row's absmax is 448): exact E4M3 values keep
    their codes, and values half way between two codes go to the even code."""
    vals = [448.0, 0.5, 1.5, 3.25, -2.0,
            1.0625,      # between 1.0 (0x38) and 1.125 (0x39): even -> 0x38
            1.1875,      # between 1.125 (0x39) and 1.25 (0x3A): even -> 0x3A
            1.5 * 2 ** -9,   # between codes 1 and 2 (subnormals): even -> 0x02
            7.5 * 2 ** -9,   # between the largest subnormal 0x07 and 2^-6 (0x08): -> 0x08
            432.0]       # between 416 (0x7D) and 448 (0x7E): even -> 0x7E
    want = [0x7E, 0x30, 0x3C, 0x45, 0xC0, 0x38, 0x3A, 0x02, 0x08, 0x7E]
    codes, scale = oracle.quantize_e4m3(np.array([vals], dtype=np.float32))
    assert scale[0] == 1.0
    assert codes[0].tolist() == want


def test_quantize_decode_roundtrip_is_identity():
    """Every finite code decoded (scale 1: the row holds 448) quantises back to itself."""
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = np.array([[oracle.e4m3_to_double(c) for c in finite]], dtype=np.float32)
    codes, scale = oracle.quantize_e4m3(vals)
    assert scale[0] == 1.0
    got = codes[0].tolist()
    for c, q in zip(finite, got):
        assert q == c or (c == 0x80 and q == 0x80), (hex(c), hex(q))


def test_quantize_bf16_input_matches_float_input():
    g = np.random.default_rng(12)
    x = torch.from_numpy(g.standard_normal((4, 256)).astype(np.float32)).to(torch.bfloat16)
    c1, s1 = oracle.quantize_e4m3(x, oracle.BF16)
    c2, s2 = oracle.quantize_e4m3(x.float().numpy(), oracle.F32)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


# ------------------------------------------------------------------ training side
#
# The backward and the indexer loss are pinned to torch's float64 autograd of the
# forward formulas (library differentiation, independent of the oracle's hand-written
# gradients), to central finite differences of the oracle's own (separately pinned)
# forward, and to closed forms.

def _train_case(rng, T, Tk, Hq, G, d, kk, pad=True):
    """f32 inputs on a 2^-6 grid (so small perturbations stay exact), causal-looking index
    lists with -1 padding."""
    q = (rng.integers(-64, 65, (T, Hq, d)) / 64.0).astype(np.float32)
    k = (rng.integers(-64, 65, (Tk, G, d)) / 64.0).astype(np.float32)
    v = (rng.integers(-64, 65, (Tk, G, d)) / 64.0).astype(np.float32)
    idx = np.full((T, kk), -1, dtype=np.int32)
    for t in range(T):
        n = rng.integers(1, kk + 1) if pad else kk
        idx[t, :n] = np.sort(rng.choice(Tk, size=n, replace=False))
    return q, k, v, idx


def _torch_attn(q, k, v, idx, G, sm_scale):
    """out [T,Hq,d] of float64 torch tensors (autograd-able) by gather + masked softmax."""
    T, Hq, d = q.shape
    hpg = Hq // G
    valid = torch.from_numpy(idx >= 0)
    ii = torch.from_numpy(np.maximum(idx, 0)).long()
    kg = k[ii]                                     # [T, kk, G, d]
    vg = v[ii]
    g_of_h = torch.arange(Hq) // hpg
    kh = kg[:, :, g_of_h, :]                       # [T, kk, Hq, d]
    vh = vg[:, :, g_of_h, :]
    logits = sm_scale * torch.einsum("thd,tkhd->thk", q, kh)
    logits = logits.masked_fill(~valid[:, None, :], float("-inf"))
    p = torch.softmax(logits, dim=-1)
    return torch.einsum("thk,tkhd->thd", p, vh), p, logits


def test_attn_lse_matches_torch_logsumexp():
    rng = np.random.default_rng(41)
    q, k, v, idx = _train_case(rng, T=6, Tk=9, Hq=4, G=2, d=8, kk=5)
    out, lse = oracle.attn_lse(q, k, v, oracle.F32, idx, 2, 0.35)
    o_t, _, logits = _torch_attn(*(torch.from_numpy(a).double() for a in (q, k, v)), idx, 2, 0.35)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, dim=-1).numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, o_t.numpy(), rtol=0, atol=1e-12)
    # a single selected position: lse is its logit and the output its V row
    one = np.full_like(idx, -1)
    one[:, 0] = 3
    out1, lse1 = oracle.attn_lse(q, k, v, oracle.F32, one, 2, 0.35)
    np.testing.assert_allclose(out1[:, :2], np.broadcast_to(v[3, 0], (6, 2, 8)), atol=1e-12)
    np.testing.assert_allclose(lse1[:, 0], 0.35 * np.einsum("td,d->t", q[:, 0].astype(np.float64),
                                                            k[3, 0].astype(np.float64)), atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attn_bwd_matches_autograd(dtype):
    rng = np.random.default_rng(42)
    T, Tk, Hq, G, d, kk, sm = 7, 11, 8, 2, 16, 6, 0.3
    q, k, v, idx = _train_case(rng, T, Tk, Hq, G, d, kk)
    dout = (rng.integers(-64, 65, (T, Hq, d)) / 64.0).astype(np.float32)
    arrs = [q, k, v, dout]
    if dtype == "bf16":                            # grid values are exact in bf16
        arrs = [torch.from_numpy(a).bfloat16() for a in arrs]
        od = oracle.BF16
    else:
        od = oracle.F32
    dq, dk, dv = oracle.attn_bwd(arrs[0], arrs[1], arrs[2], od, idx, G, sm, arrs[3])
    qt, kt, vt = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    out, _, _ = _torch_attn(qt, kt, vt, idx, G, sm)
    (out * torch.from_numpy(dout).double()).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-11)
    # positions nobody selected get no gradient
    unused = np.setdiff1d(np.arange(Tk), idx[idx >= 0])
    assert np.all(dk[unused] == 0) and np.all(dv[unused] == 0)


def test_attn_bwd_central_differences_of_the_forward():
    rng = np.random.default_rng(43)
    T, Tk, Hq, G, d, kk, sm = 4, 6, 4, 2, 8, 4, 0.5
    q, k, v, idx = _train_case(rng, T, Tk, Hq, G, d, kk, pad=False)
    dout = (rng.integers(-64, 65, (T, Hq, d)) / 64.0)
    dq, dk, dv = oracle.attn_bwd(q, k, v, oracle.F32, idx, G, sm, dout.astype(np.float32))

    def loss(q_, k_, v_):
        return float((oracle.sparse_gqa_attn(q_, k_, v_, oracle.F32, idx, Hq, G, sm) * dout).sum())
    h = 2.0 ** -10
    for arr, grad, pos in ((q, dq, (1, 2, 3)), (k, dk, (int(idx[0, 1]), 1, 5)),
                           (v, dv, (int(idx[2, 0]), 0, 7))):
        plus, minus = arr.copy(), arr.copy()
        plus[pos] += h
        minus[pos] -= h
        args_p = [plus if a is arr else a for a in (q, k, v)]
        args_m = [minus if a is arr else a for a in (q, k, v)]
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert abs(fd - grad[pos]) <= 1e-5 * max(1.0, abs(fd)), (pos, fd, grad[pos])


def _torch_kl(q, k, idx, G, sm, vals):
    """kl [T] from torch float64 (vals autograd-able)."""
    T, Hq, d = q.shape
    qd, kd = torch.from_numpy(q).double(), torch.from_numpy(k).double()
    _, p, _ = _torch_attn(qd, kd, kd, idx, G, sm)          # v unused
    pg = p.view(T, G, Hq // G, -1).mean(dim=2)              # [T, G, kk]
    valid = torch.from_numpy(idx >= 0)
    logq = torch.log_softmax(vals.masked_fill(~valid, float("-inf")), dim=-1)
    logq = logq.masked_fill(~valid, 0.0)
    terms = torch.special.xlogy(pg, pg) - pg * logq[:, None, :]
    return terms.sum(dim=(1, 2))


def test_indexer_kl_matches_autograd():
    rng = np.random.default_rng(44)
    T, Tk, Hq, G, d, kk, sm = 6, 10, 8, 4, 8, 7, 0.4
    q, k, _, idx = _train_case(rng, T, Tk, Hq, G, d, kk)
    vals = rng.normal(size=(T, kk))
    vals[idx < 0] = -np.inf
    kl, dI = oracle.indexer_kl(q, k, oracle.F32, idx, G, sm, vals)
    vt = torch.tensor(np.where(idx >= 0, vals, 0.0), requires_grad=True)
    kt = _torch_kl(q, k, idx, G, sm, vt)
    kt.sum().backward()
    np.testing.assert_allclose(kl, kt.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dI, np.where(idx >= 0, vt.grad.numpy(), 0.0), rtol=0, atol=1e-12)
    assert np.all(kl >= -1e-12)                    # a KL divergence is never negative
    np.testing.assert_allclose(dI.sum(axis=1), 0.0, atol=1e-12)   # softmax gradients sum to 0


def test_indexer_kl_vanishes_when_the_indexer_matches_the_target():
    """One KV group: the target is the mean head distribution; scores equal to its log
    (plus any constant) give KL = 0 and a zero gradient."""
    rng = np.random.default_rng(45)
    T, Tk, Hq, G, d, kk, sm = 5, 9, 4, 1, 8, 6, 0.7
    q, k, _, idx = _train_case(rng, T, Tk, Hq, G, d, kk)
    _, p, _ = _torch_attn(torch.from_numpy(q).double(), torch.from_numpy(k).double(),
                          torch.from_numpy(k).double(), idx, G, sm)
    target = p.mean(dim=1).numpy()                              # [T, kk]
    vals = np.where(idx >= 0, np.log(np.maximum(target, 1e-300)) + 3.25, -np.inf)
    kl, dI = oracle.indexer_kl(q, k, oracle.F32, idx, G, sm, vals)
    np.testing.assert_allclose(kl, 0.0, atol=1e-12)
    np.testing.assert_allclose(dI, 0.0, atol=1e-12)


def _torch_indexer(qi, w, ki, idx):
    """I[t, idx[t,i]] in float64 torch from dequantised inputs (autograd-able)."""
    ii = torch.from_numpy(np.maximum(idx, 0)).long()
    kg = ki[ii]                                            # [T, kk, dI]
    x = torch.einsum("tjd,tkd->tjk", qi, kg)              # [T, HI, kk]
    return (w[:, :, None] * torch.relu(x)).sum(dim=1)     # [T, kk]


@pytest.mark.parametrize("fp8", [False, True])
def test_indexer_scores_at_and_backward_match_autograd(fp8):
    rng = np.random.default_rng(46)
    T, Tk, HI, dI, kk = 5, 12, 4, 8, 6
    _, _, _, idx = _train_case(rng, T, Tk, 2, 1, 4, kk)
    w = rng.normal(size=(T, HI)).astype(np.float32)         # signed weights
    if fp8:
        qc = rng.integers(0, 256, (T, HI, dI), dtype=np.uint8)
        kc = rng.integers(0, 256, (Tk, dI), dtype=np.uint8)
        qc[(qc & 0x7F) == 0x7F] = 0x38                       # no NaN codes
        kc[(kc & 0x7F) == 0x7F] = 0x38
        qs = rng.uniform(0.01, 0.1, T).astype(np.float32)
        ks = rng.uniform(0.01, 0.1, Tk).astype(np.float32)
        lut = np.array([oracle.e4m3_to_double(c) for c in range(256)])
        qd, kd = lut[qc] * qs[:, None, None], lut[kc] * ks[:, None]
        args = (qc, qs, w, kc, ks, oracle.FP8_E4M3)
    else:
        qd = rng.normal(size=(T, HI, dI)).astype(np.float32)
        kd = rng.normal(size=(Tk, dI)).astype(np.float32)
        args = (qd, None, w, kd, None, oracle.F32)
    vals = oracle.index_scores_at(*args, idx)
    g = rng.normal(size=(T, kk))
    dq, dw, dk = oracle.index_scores_bwd(*args, idx, g)
    qt = torch.tensor(np.asarray(qd, dtype=np.float64), requires_grad=True)
    kt = torch.tensor(np.asarray(kd, dtype=np.float64), requires_grad=True)
    wt = torch.tensor(w.astype(np.float64), requires_grad=True)
    It = _torch_indexer(qt, wt, kt, idx)
    valid = idx >= 0
    np.testing.assert_allclose(np.where(valid, vals, 0), np.where(valid, It.detach().numpy(), 0),
                               rtol=1e-12, atol=1e-12)
    assert np.all(vals[~valid] == -np.inf)
    (It * torch.from_numpy(np.where(valid, g, 0.0))).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_indexer_scores_at_equal_full_rows_gathered():
    rng = np.random.default_rng(47)
    T, HI, dI, k = 40, 8, 128, 16
    qc, qs, w, kc, ks = _rand_fp8_case(rng, T, HI, dI)
    full = oracle.index_scores(qc, qs, w, kc, ks, oracle.FP8_E4M3)
    idx, _ = oracle.topk(full, np.arange(T, dtype=np.int64), k)
    vals = oracle.index_scores_at(qc, qs, w, kc, ks, oracle.FP8_E4M3, idx)
    valid = idx >= 0
    np.testing.assert_allclose(vals[valid], np.take_along_axis(full, np.maximum(idx, 0), 1)[valid],
                               rtol=1e-13, atol=1e-13)


# ------------------------------------------------- dense warm-up indexer loss

def _dense_case(rng, T, Tk, Hq, G, d, q_pos0):
    q = (rng.integers(-64, 65, (T, Hq, d)) / 64.0).astype(np.float32)
    k = (rng.integers(-64, 65, (Tk, G, d)) / 64.0).astype(np.float32)
    pos = q_pos0 + np.arange(T)
    causal = np.arange(Tk)[None, :] <= pos[:, None]          # [T, Tk]
    scores = np.where(causal, rng.normal(size=(T, Tk)), -np.inf)
    return q, k, causal, scores


def test_warmup_kl_matches_dense_masked_softmax_autograd():
    """Every row against torch float64 over the full causal score matrix: a masked softmax per
    head, the mean over each group's heads, the log-softmax of I, and autograd for dI."""
    rng = np.random.default_rng(48)
    T, Tk, Hq, G, d, q_pos0, sm = 6, 11, 8, 4, 8, 4, 0.45
    q, k, causal, scores = _dense_case(rng, T, Tk, Hq, G, d, q_pos0)
    kl, dI = oracle.indexer_warmup_kl(q, k, oracle.F32, G, sm, scores, q_pos0=q_pos0)
    qd, kd = torch.from_numpy(q).double(), torch.from_numpy(k).double()
    hpg = Hq // G
    kh = kd[:, torch.arange(Hq) // hpg, :]                     # [Tk, Hq, d]
    logits = sm * torch.einsum("thd,shd->ths", qd, kh)         # [T, Hq, Tk]
    mask = torch.from_numpy(causal)
    P = torch.softmax(logits.masked_fill(~mask[:, None, :], float("-inf")), dim=-1)
    pg = P.view(T, G, hpg, Tk).mean(dim=2)                     # [T, G, Tk]
    It = torch.tensor(np.where(causal, scores, 0.0), requires_grad=True)
    logq = torch.log_softmax(It.masked_fill(~mask, float("-inf")), dim=-1).masked_fill(~mask, 0.0)
    loss = (torch.special.xlogy(pg, pg) - pg * logq[:, None, :]).sum(dim=(1, 2))
    loss.sum().backward()
    np.testing.assert_allclose(kl, loss.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dI, np.where(causal, It.grad.numpy(), 0.0), rtol=0, atol=1e-12)
    assert np.all(dI[~causal] == 0.0)
    np.testing.assert_allclose(dI.sum(axis=1), 0.0, atol=1e-12)


def test_warmup_kl_uniform_target_closed_form():
    """q = 0 makes every head attend uniformly to the n = pos + 1 keys of its prefix, so
    KL[t] = G (-ln n - mean_s log softmax(I)_s) and dI = G (softmax(I) - 1/n); equal scores
    then give KL = 0."""
    rng = np.random.default_rng(49)
    T, Tk, Hq, G, d, q_pos0, sm = 5, 9, 4, 2, 8, 2, 1.3
    q, k, causal, scores = _dense_case(rng, T, Tk, Hq, G, d, q_pos0)
    q[:] = 0.0
    kl, dI = oracle.indexer_warmup_kl(q, k, oracle.F32, G, sm, scores, q_pos0=q_pos0)
    for t in range(T):
        n = q_pos0 + t + 1
        row = scores[t, :n]
        ls = row - row.max() - math.log(np.exp(row - row.max()).sum())
        assert kl[t] == pytest.approx(G * (-math.log(n) - ls.mean()), rel=1e-12, abs=1e-12)
        np.testing.assert_allclose(dI[t, :n], G * (np.exp(ls) - 1.0 / n), rtol=0, atol=1e-13)
    flat = np.where(causal, 2.5, -np.inf)
    kl0, dI0 = oracle.indexer_warmup_kl(q, k, oracle.F32, G, sm, flat, q_pos0=q_pos0)
    np.testing.assert_allclose(kl0, 0.0, atol=1e-12)
    np.testing.assert_allclose(dI0, 0.0, atol=1e-12)


@pytest.mark.parametrize("fp8", [False, True])
def test_index_scores_bwd_dense_matches_autograd(fp8):
    """The dense indexer backward against torch float64 autograd of the whole score matrix
    I[t, s] = sum_j w ReLU(q^I_j . k^I_s), with g applied on the causal part only."""
    rng = np.random.default_rng(50)
    T, Tk, HI, dI, q_pos0 = 5, 10, 4, 8, 3
    w = rng.normal(size=(T, HI)).astype(np.float32)
    if fp8:
        qc = rng.integers(0, 256, (T, HI, dI), dtype=np.uint8)
        kc = rng.integers(0, 256, (Tk, dI), dtype=np.uint8)
        qc[(qc & 0x7F) == 0x7F] = 0x38
        kc[(kc & 0x7F) == 0x7F] = 0x38
        qs = rng.uniform(0.01, 0.1, T).astype(np.float32)
        ks = rng.uniform(0.01, 0.1, Tk).astype(np.float32)
        lut = np.array([oracle.e4m3_to_double(c) for c in range(256)])
        qd, kd = lut[qc] * qs[:, None, None], lut[kc] * ks[:, None]
        args = (qc, qs, w, kc, ks, oracle.FP8_E4M3)
    else:
        qd = rng.normal(size=(T, HI, dI)).astype(np.float32)
        kd = rng.normal(size=(Tk, dI)).astype(np.float32)
        args = (qd, None, w, kd, None, oracle.F32)
    causal = np.arange(Tk)[None, :] <= (q_pos0 + np.arange(T))[:, None]
    g = rng.normal(size=(T, Tk))
    dq, dw, dk = oracle.index_scores_bwd_dense(*args, g, q_pos0=q_pos0)
    qt = torch.tensor(np.asarray(qd, dtype=np.float64), requires_grad=True)
    kt = torch.tensor(np.asarray(kd, dtype=np.float64), requires_grad=True)
    wt = torch.tensor(w.astype(np.float64), requires_grad=True)
    It = (wt[:, :, None] * torch.relu(torch.einsum("tjd,sd->tjs", qt, kt))).sum(dim=1)
    (It * torch.from_numpy(np.where(causal, g, 0.0))).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_indexer_kl_finite_when_scores_lie_far_below_the_max():
    """A score 1000 below the row's best makes exp underflow in double; the divergence is
    still the finite value of the definition.  q = 0 (uniform target over the two keys):
    KL = G (-ln 2 - (1/2) sum_s log softmax(I)_s) with log softmax = (-ln(1 + e^-1000), -1000)."""
    T, Tk, Hq, G, d, sm = 2, 2, 4, 2, 8, 1.0
    q = np.zeros((T, Hq, d), dtype=np.float32)
    k = np.ones((Tk, G, d), dtype=np.float32)
    scores = np.array([[0.0, -np.inf], [0.0, -1000.0]])
    kl, dI = oracle.indexer_warmup_kl(q, k, oracle.F32, G, sm, scores)
    assert kl[0] == 0.0
    assert kl[1] == pytest.approx(G * (-math.log(2.0) + 500.0), rel=1e-14)
    np.testing.assert_allclose(dI[1], [G * (1.0 - 0.5), G * (0.0 - 0.5)], atol=1e-15)
    idx = np.array([[0, -1], [0, 1]], dtype=np.int32)
    kl2, _ = oracle.indexer_kl(q, k, oracle.F32, idx, G, sm, np.where(idx >= 0, scores, -np.inf))
    assert np.isfinite(kl2).all() and kl2[1] == pytest.approx(kl[1], rel=1e-14)
