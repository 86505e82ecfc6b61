"""CPU oracle for the DSA layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The GPU library never does, and it
shares no code with the C source here (``oracle.c``).

The functions follow the formulas of the Kwai Keye-VL-2.0 report (xllm-io
review page, section "核心公式"; report section 2.3): the lightning indexer
score, the Top-k index set and GQA sparse aggregation, and on the training
side (``oracle_train.c``; report section 2.3.3 and the review page's sparse
adaptation and dense warm-up losses) the attention backward and both indexer
losses.  Every
result is float64.  See the C sources for the arithmetic and the readings of
points the pages leave open.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SRC_TRAIN = os.path.join(_HERE, "oracle_train.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8_E4M3 = 0, 1, 2

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with the host C compiler (no -ffast-math)."""
    newest = max(os.path.getmtime(p) for p in (_SRC, _SRC_TRAIN, os.path.join(_HERE, "oracle.h")))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, _SRC_TRAIN, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
            lib.oracle_e4m3_to_double.restype = D
            lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
            lib.oracle_bf16_to_double.restype = D
            lib.oracle_index_scores.argtypes = [P, P, P, P, P, I, I, I, I, I, I64, P, I, P]
            lib.oracle_index_scores.restype = None
            lib.oracle_topk.argtypes = [P, I64, I, P, I, P, P]
            lib.oracle_topk.restype = None
            lib.oracle_sparse_gqa_attn.argtypes = [P, P, P, I, P, I, I, P, P, I, P, I, I, I, I, D, P]
            lib.oracle_sparse_gqa_attn.restype = None
            lib.oracle_decode.argtypes = [P, P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I,
                                          I, D, P, I, P, P, P]
            lib.oracle_decode.restype = None
            lib.oracle_quantize_e4m3.argtypes = [P, I, I, I, P, P]
            lib.oracle_quantize_e4m3.restype = None
            lib.oracle_attn_lse.argtypes = [P, P, P, I, P, I, I, I, I, I, D, P, P]
            lib.oracle_attn_lse.restype = None
            lib.oracle_attn_bwd.argtypes = [P, P, P, I, P, I, I, I, I, I, I, D, P, P, P, P]
            lib.oracle_attn_bwd.restype = None
            lib.oracle_indexer_kl.argtypes = [P, P, I, P, I, I, I, I, I, D, P, P, P]
            lib.oracle_indexer_kl.restype = None
            lib.oracle_indexer_warmup_kl.argtypes = [P, P, I, I, I, I64, I, I, I, D, P, P, P]
            lib.oracle_indexer_warmup_kl.restype = None
            lib.oracle_index_scores_bwd_dense.argtypes = [P, P, P, P, P, I, I, I, I, I, I64, P, P,
                                                          P, P]
            lib.oracle_index_scores_bwd_dense.restype = None
            lib.oracle_index_scores_at.argtypes = [P, P, P, P, P, I, I, I, I, P, I, P]
            lib.oracle_index_scores_at.restype = None
            lib.oracle_index_scores_bwd.argtypes = [P, P, P, P, P, I, I, I, I, I, P, I, P, P, P, P]
            lib.oracle_index_scores_bwd.restype = None
            lib.oracle_num_threads.argtypes = []
            lib.oracle_num_threads.restype = I
            _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _np(a, dtype=None):
    """Accept numpy arrays or CPU torch tensors; return a C-contiguous numpy array."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        t = a.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.uint16)
        elif t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        a = t.numpy()
    a = np.ascontiguousarray(a)
    if dtype is not None and a.dtype != dtype:
        a = a.astype(dtype)
    return a


def num_threads() -> int:
    return _load().oracle_num_threads()


def e4m3_to_double(code: int) -> float:
    return _load().oracle_e4m3_to_double(code)


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(bits)


def index_scores(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, q_pos0=0, rows=None):
    """I[t, s] for the query rows ``rows`` (default: all), s in [0, Tk).

    q_idx [Tq, HI, dI] (uint8 E4M3 codes or float32), q_scale [Tq] or None,
    w [Tq, HI] float32, k_idx [Tk, dI], k_scale [Tk] or None.  Entries with
    s > q_pos0 + t are -inf.  Returns float64 [len(rows), Tk].
    """
    lib = _load()
    code_dtype = np.uint8 if idx_dtype == FP8_E4M3 else np.float32
    q_idx = _np(q_idx, code_dtype)
    k_idx = _np(k_idx, code_dtype)
    w = _np(w, np.float32)
    q_scale = _np(q_scale, np.float32)
    k_scale = _np(k_scale, np.float32)
    Tq, HI, dI = q_idx.shape
    Tk = k_idx.shape[0]
    assert k_idx.shape == (Tk, dI) and w.shape == (Tq, HI)
    if idx_dtype == FP8_E4M3:
        assert q_scale.shape == (Tq,) and k_scale.shape == (Tk,)
    rows = np.arange(Tq, dtype=np.int32) if rows is None else _np(rows, np.int32)
    out = np.empty((len(rows), Tk), dtype=np.float64)
    lib.oracle_index_scores(_ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale),
                            idx_dtype, Tq, Tk, HI, dI, int(q_pos0), _ptr(rows), len(rows),
                            _ptr(out))
    return out


def topk(scores, pos, k):
    """Top-k of each row of ``scores`` over candidates 0..pos[r].

    Returns (idx int32 [rows, k] ascending with -1 padding, kth float64 [rows]):
    kth is the score of the last member in selection order (the k-th largest,
    or the smallest when fewer than k candidates exist).
    """
    lib = _load()
    scores = _np(scores, np.float64)
    if scores.ndim == 1:
        scores = scores[None, :]
    pos = _np(np.broadcast_to(np.asarray(pos, dtype=np.int64), (scores.shape[0],)), np.int64)
    assert np.all(pos < scores.shape[1])
    idx = np.empty((scores.shape[0], k), dtype=np.int32)
    kth = np.empty(scores.shape[0], dtype=np.float64)
    lib.oracle_topk(_ptr(scores), scores.shape[1], scores.shape[0], _ptr(pos), k, _ptr(idx),
                    _ptr(kth))
    return idx, kth


def sparse_gqa_attn(q, k, v, dtype, idx, Hq, G, sm_scale, rows=None, block_table=None,
                    block_size=0, row_seq=None):
    """Attention of each query row over its index set (same set for every group).

    q [T, Hq, d]; k, v [Tk, G, d] (or paged [NB, block_size, G, d] with
    block_table [B, max_blocks] and row_seq [T]); idx [T, kk] (-1 skipped).
    dtype: F32 or BF16 (bf16 passed as uint16 bits).  Returns float64
    [len(rows), Hq, d].
    """
    lib = _load()
    el = np.float32 if dtype == F32 else np.uint16
    q, k, v = _np(q, el), _np(k, el), _np(v, el)
    idx = _np(idx, np.int32)
    T, Hq_, d = q.shape
    assert Hq_ == Hq and Hq % G == 0
    kk = idx.shape[1]
    rows = np.arange(T, dtype=np.int32) if rows is None else _np(rows, np.int32)
    bt = _np(block_table, np.int32)
    rs = _np(row_seq, np.int32)
    max_blocks = 0 if bt is None else bt.shape[1]
    out = np.empty((len(rows), Hq, d), dtype=np.float64)
    lib.oracle_sparse_gqa_attn(_ptr(q), _ptr(k), _ptr(v), dtype, _ptr(bt), max_blocks,
                               int(block_size), _ptr(rs), _ptr(idx), kk, _ptr(rows), len(rows),
                               Hq, G, d, float(sm_scale), _ptr(out))
    return out


def decode(q, q_idx, q_scale, w, kidx_cache, kidx_scale, k_cache, v_cache, dtype,
           block_table, seq_lens, block_size, k, sm_scale, seqs=None):
    """One paged decode step for the sequences ``seqs`` (default: all).

    Returns (idx int32 [n, k], kth float64 [n], out float64 [n, Hq, d]).
    """
    lib = _load()
    el = np.float32 if dtype == F32 else np.uint16
    q = _np(q, el)
    q_idx = _np(q_idx, np.uint8)
    q_scale, w = _np(q_scale, np.float32), _np(w, np.float32)
    kidx_cache, kidx_scale = _np(kidx_cache, np.uint8), _np(kidx_scale, np.float32)
    k_cache, v_cache = _np(k_cache, el), _np(v_cache, el)
    block_table, seq_lens = _np(block_table, np.int32), _np(seq_lens, np.int32)
    B, Hq, d = q.shape
    _, HI, dI = q_idx.shape
    G = k_cache.shape[2]
    seqs = np.arange(B, dtype=np.int32) if seqs is None else _np(seqs, np.int32)
    n = len(seqs)
    idx = np.empty((n, k), dtype=np.int32)
    kth = np.empty(n, dtype=np.float64)
    out = np.empty((n, Hq, d), dtype=np.float64)
    lib.oracle_decode(_ptr(q), _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(kidx_cache),
                      _ptr(kidx_scale), _ptr(k_cache), _ptr(v_cache), dtype, _ptr(block_table),
                      _ptr(seq_lens), block_table.shape[1], int(block_size), HI, dI, Hq, G, d,
                      int(k), float(sm_scale), _ptr(seqs), n, _ptr(idx), _ptr(kth), _ptr(out))
    return idx, kth, out


def quantize_e4m3(x, x_dtype=F32):
    """Per-token E4M3 codes and scales of x [T, ...] (F32 or BF16 input).

    Returns (codes uint8 of x's shape, scale float32 [T])."""
    lib = _load()
    x = _np(x, np.float32 if x_dtype == F32 else np.uint16)
    T = x.shape[0]
    n = int(np.prod(x.shape[1:])) if x.ndim > 1 else 1
    codes = np.empty(x.shape, dtype=np.uint8)
    scale = np.empty(T, dtype=np.float32)
    lib.oracle_quantize_e4m3(_ptr(x), x_dtype, T, n, _ptr(codes), _ptr(scale))
    return codes, scale


# ------------------------------------------------------------------ training side

def _attn_arrays(q, k, v, dtype, idx):
    el = np.float32 if dtype == F32 else np.uint16
    return _np(q, el), _np(k, el), (None if v is None else _np(v, el)), _np(idx, np.int32)


def attn_lse(q, k, v, dtype, idx, G, sm_scale):
    """(out float64 [T, Hq, d], lse float64 [T, Hq]) of the attention over idx."""
    lib = _load()
    q, k, v, idx = _attn_arrays(q, k, v, dtype, idx)
    T, Hq, d = q.shape
    out = np.empty((T, Hq, d), dtype=np.float64)
    lse = np.empty((T, Hq), dtype=np.float64)
    lib.oracle_attn_lse(_ptr(q), _ptr(k), _ptr(v), dtype, _ptr(idx), idx.shape[1], T, Hq, G, d,
                        float(sm_scale), _ptr(out), _ptr(lse))
    return out, lse


def attn_bwd(q, k, v, dtype, idx, G, sm_scale, dout):
    """(dq [T,Hq,d], dk [Tk,G,d], dv [Tk,G,d]) float64: gradients of sum(dout * out)."""
    lib = _load()
    q, k, v, idx = _attn_arrays(q, k, v, dtype, idx)
    dout = _np(dout, np.float32 if dtype == F32 else np.uint16)
    T, Hq, d = q.shape
    Tk = k.shape[0]
    dq = np.empty((T, Hq, d), dtype=np.float64)
    dk = np.empty((Tk, G, d), dtype=np.float64)
    dv = np.empty((Tk, G, d), dtype=np.float64)
    lib.oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), dtype, _ptr(idx), idx.shape[1], T, Tk, Hq, G,
                        d, float(sm_scale), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def indexer_kl(q, k, dtype, idx, G, sm_scale, vals):
    """(kl float64 [T], dI float64 [T, kk]) of the sparse indexer loss."""
    lib = _load()
    q, k, _, idx = _attn_arrays(q, k, None, dtype, idx)
    T, Hq, d = q.shape
    vals = np.ascontiguousarray(np.asarray(vals, dtype=np.float64))
    kl = np.empty(T, dtype=np.float64)
    dI = np.empty(idx.shape, dtype=np.float64)
    lib.oracle_indexer_kl(_ptr(q), _ptr(k), dtype, _ptr(idx), idx.shape[1], T, Hq, G, d,
                          float(sm_scale), _ptr(vals), _ptr(kl), _ptr(dI))
    return kl, dI


def indexer_warmup_kl(q, k, dtype, G, sm_scale, scores, q_pos0=0):
    """(kl float64 [T], dI float64 [T, Tk]) of the dense warm-up indexer loss: row t at
    position q_pos0 + t, its set every key s <= q_pos0 + t; scores [T, Tk] = I[t, s]."""
    lib = _load()
    q, k, _, _ = _attn_arrays(q, k, None, dtype, np.zeros((1, 1), np.int32))
    T, Hq, d = q.shape
    scores = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    Tk = scores.shape[1]
    assert scores.shape[0] == T and k.shape[0] >= Tk
    kl = np.empty(T, dtype=np.float64)
    dI = np.empty((T, Tk), dtype=np.float64)
    lib.oracle_indexer_warmup_kl(_ptr(q), _ptr(k), dtype, T, Tk, int(q_pos0), Hq, G, d,
                                 float(sm_scale), _ptr(scores), _ptr(kl), _ptr(dI))
    return kl, dI


def _indexer_arrays(q_idx, q_scale, w, k_idx, k_scale, idx_dtype):
    el = np.uint8 if idx_dtype == FP8_E4M3 else np.float32
    return (_np(q_idx, el), _np(q_scale, np.float32), _np(w, np.float32), _np(k_idx, el),
            _np(k_scale, np.float32))


def index_scores_at(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, idx):
    """vals float64 [T, kk] = I[t, idx[t, i]] (-inf for padding)."""
    lib = _load()
    q_idx, q_scale, w, k_idx, k_scale = _indexer_arrays(q_idx, q_scale, w, k_idx, k_scale, idx_dtype)
    idx = _np(idx, np.int32)
    T, HI, dI = q_idx.shape
    vals = np.empty(idx.shape, dtype=np.float64)
    lib.oracle_index_scores_at(_ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale),
                               idx_dtype, T, HI, dI, _ptr(idx), idx.shape[1], _ptr(vals))
    return vals


def index_scores_bwd(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, idx, g):
    """(dq_idx [T,HI,dI], dw [T,HI], dk_idx [Tk,dI]) float64: gradients of
    sum g[t,i] * I[t, idx[t,i]] with respect to the dequantised indexer inputs."""
    lib = _load()
    q_idx, q_scale, w, k_idx, k_scale = _indexer_arrays(q_idx, q_scale, w, k_idx, k_scale, idx_dtype)
    idx = _np(idx, np.int32)
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float64))
    T, HI, dI = q_idx.shape
    Tk = k_idx.shape[0]
    dq = np.empty((T, HI, dI), dtype=np.float64)
    dw = np.empty((T, HI), dtype=np.float64)
    dk = np.empty((Tk, dI), dtype=np.float64)
    lib.oracle_index_scores_bwd(_ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale),
                                idx_dtype, T, Tk, HI, dI, _ptr(idx), idx.shape[1], _ptr(g),
                                _ptr(dq), _ptr(dw), _ptr(dk))
    return dq, dw, dk


def index_scores_bwd_dense(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, g, q_pos0=0):
    """(dq_idx, dw, dk_idx) float64 for a dense g [T, Tk]: gradients of
    sum_{t, s <= q_pos0 + t} g[t,s] * I[t,s]."""
    lib = _load()
    q_idx, q_scale, w, k_idx, k_scale = _indexer_arrays(q_idx, q_scale, w, k_idx, k_scale, idx_dtype)
    g = np.ascontiguousarray(np.asarray(g, dtype=np.float64))
    T, HI, dI = q_idx.shape
    Tk = g.shape[1]
    assert g.shape[0] == T and k_idx.shape[0] >= Tk
    dq = np.empty((T, HI, dI), dtype=np.float64)
    dw = np.empty((T, HI), dtype=np.float64)
    dk = np.empty((Tk, dI), dtype=np.float64)
    lib.oracle_index_scores_bwd_dense(_ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx),
                                      _ptr(k_scale), idx_dtype, T, Tk, HI, dI, int(q_pos0),
                                      _ptr(g), _ptr(dq), _ptr(dw), _ptr(dk))
    return dq, dw, dk
