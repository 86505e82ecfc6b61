"""libdsa: DeepSeek Sparse Attention (GQA form) for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/dsa.h``.  Every step of the
layer -- lightning indexer, top-k, GQA sparse attention, the fused prefill and
paged decode -- runs in the HIP kernels of ``libdsa.so``; this module only
marshals torch tensors (device pointers) and the current HIP stream.  It has
no fallback: if the library is missing or the tensors are not on the GPU the
calls raise.

Functions named ``dsa_*`` mirror the C entry points one to one.  ``prefill``
and ``decode`` are conveniences that allocate outputs and workspace with torch
and call ``dsa_prefill`` / ``dsa_decode``; ``quantize_e4m3`` and ``cache_append``
do the same for the step before decode.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
          4: "DSA_ERR_HIP"}

# every symbol the header declares, in declaration order
EXPORTS = ["dsa_status_string", "dsa_last_error", "dsa_version",
           "dsa_index_scores_workspace_size", "dsa_index_scores",
           "dsa_topk_workspace_size", "dsa_topk", "dsa_sparse_gqa_attn_workspace_size",
           "dsa_sparse_gqa_attn", "dsa_sparse_gqa_attn_dedup_workspace_size",
           "dsa_sparse_gqa_attn_dedup", "dsa_prefill_workspace_size", "dsa_prefill_stats_offset",
           "dsa_prefill", "dsa_prefill_varlen", "dsa_decode_workspace_size", "dsa_decode_stats_offset", "dsa_decode",
           "dsa_decode_noalloc_max_workspace", "dsa_decode_noalloc",
           "dsa_quantize_e4m3", "dsa_cache_append", "dsa_index_scores_at",
           "dsa_index_scores_at_bwd_workspace_size", "dsa_index_scores_at_bwd", "dsa_sparse_gqa_attn_lse", "dsa_sparse_gqa_attn_bwd_workspace_size",
           "dsa_sparse_gqa_attn_bwd", "dsa_indexer_warmup_kl",
           "dsa_index_scores_bwd_dense_workspace_size", "dsa_index_scores_bwd_dense"]


class DSAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), detail))
        self.status = status
        self.detail = detail


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so (built in-tree by ``build.build()``); raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise OSError("libdsa.so not found at %s; build it with "
                          "`python -m long_context_sparse_02_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, I, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
        sig = {
            "dsa_status_string": ([I], ctypes.c_char_p),
            "dsa_last_error": ([], ctypes.c_char_p),
            "dsa_version": ([], I),
            "dsa_index_scores_workspace_size": ([I, I, I, I], SZ),
            "dsa_index_scores": ([P, P, P, P, P, I, I, I, I, I, I64, P, I64, P, SZ, P], I),
            "dsa_topk_workspace_size": ([I, I, I], SZ),
            "dsa_topk": ([P, I64, I, I, I64, I, P, P, SZ, P], I),
            "dsa_sparse_gqa_attn_workspace_size": ([I, I, I, I], SZ),
            "dsa_sparse_gqa_attn": ([P, P, P, I, I, P, I, I, P, P, P, I, I, I, I, I, F, P, P, SZ, P], I),
            "dsa_sparse_gqa_attn_dedup_workspace_size": ([I, I64, I], SZ),
            "dsa_sparse_gqa_attn_dedup": ([P, P, P, I, P, I, I64, I, I, I, I, F, I, P, P, SZ, P],
                                          I),
            "dsa_prefill_workspace_size": ([I, I64, I, I], SZ),
            "dsa_prefill_stats_offset": ([I, I64, I, I], SZ),
            "dsa_prefill": ([P, P, P, I, P, P, P, P, P, I, I, I64, I, I, I, I, I, I, F, I, P, P, P,
                             SZ, P], I),
            "dsa_prefill_varlen": ([P, P, P, I, P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, P,
                                    P, P, SZ, P], I),
            "dsa_decode_workspace_size": ([I, I, I, I, I, I], SZ),
            "dsa_decode_stats_offset": ([I, I, I, I, I, I], SZ),
            "dsa_decode": ([P, P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, I, I, I, F, P, P,
                            P, SZ, P], I),
            "dsa_decode_noalloc_max_workspace": ([], SZ),
            "dsa_decode_noalloc": ([P, P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, I, I, I,
                                    F, P, P, P], I),
            "dsa_quantize_e4m3": ([P, I, I, I, P, P, P], I),
            "dsa_cache_append": ([P, P, I, P, I, P, P, I, I, I, I, I, I, I, P, P, P, P, P], I),
            "dsa_index_scores_at": ([P, P, P, P, P, I, I, I, I, I, P, I, P, P], I),
            "dsa_index_scores_at_bwd_workspace_size": ([I, I, I, I], SZ),
            "dsa_index_scores_at_bwd": ([P, P, P, P, P, I, I, I, I, I, P, I, P, P, P, P, P, SZ, P], I),
            "dsa_sparse_gqa_attn_lse": ([P, P, P, I, I, P, I, I, I, I, I, F, P, P, P, SZ, P], I),
            "dsa_sparse_gqa_attn_bwd_workspace_size": ([I, I, I, I], SZ),
            "dsa_sparse_gqa_attn_bwd": ([P, P, P, I, I, P, I, I, I, I, I, F, P, P, P, P, P, P, P, P,
                                         P, P, SZ, P], I),
            "dsa_indexer_warmup_kl": ([P, P, I, I, I, I64, I, I, I, F, P, P, I64, P, P], I),
            "dsa_index_scores_bwd_dense_workspace_size": ([I, I, I], SZ),
            "dsa_index_scores_bwd_dense": ([P, P, P, P, P, I, I, I, I, I, I64, P, I64, P, P, P, P,
                                            SZ, P], I),
        }
        for name in EXPORTS:
            fn = getattr(lib, name)
            fn.argtypes, fn.restype = sig[name]
        _lib = lib
        return lib


def _check(status: int):
    if status != 0:
        raise DSAError(status, load_library().dsa_last_error().decode())


def _ptr(t):
    """Device pointer of a CUDA tensor (None -> NULL).  Host tensors are rejected."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libdsa takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libdsa takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def dtype_code(t) -> int:
    import torch
    return {torch.float32: DSA_F32, torch.bfloat16: DSA_BF16, torch.uint8: DSA_FP8_E4M3,
            torch.float8_e4m3fn: DSA_FP8_E4M3}[t.dtype]


# ------------------------------------------------------------ raw entry points

def dsa_version() -> int:
    return load_library().dsa_version()


def dsa_index_scores_workspace_size(Tq, HI, dI, idx_dtype) -> int:
    return load_library().dsa_index_scores_workspace_size(Tq, HI, dI, idx_dtype)


def dsa_index_scores(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI, q_pos0, scores,
                     ld_scores, ws=None, ws_bytes=0, stream=None):
    _check(load_library().dsa_index_scores(_ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx),
                                           _ptr(k_scale), idx_dtype, Tq, Tk, HI, dI, q_pos0,
                                           _ptr(scores), ld_scores, _ptr(ws), ws_bytes,
                                           _stream(stream)))


def dsa_topk_workspace_size(Tq, Tk, k) -> int:
    return load_library().dsa_topk_workspace_size(Tq, Tk, k)


def dsa_topk(scores, ld_scores, Tq, Tk, q_pos0, k, idx, ws=None, ws_bytes=0, stream=None):
    _check(load_library().dsa_topk(_ptr(scores), ld_scores, Tq, Tk, q_pos0, k, _ptr(idx), _ptr(ws),
                                   ws_bytes, _stream(stream)))


def dsa_sparse_gqa_attn_workspace_size(Tq, k, Hq, d) -> int:
    return load_library().dsa_sparse_gqa_attn_workspace_size(Tq, k, Hq, d)


def dsa_sparse_gqa_attn(q, k, v, dtype, n_kv, block_table, max_blocks, block_size, row_seq,
                        seq_lens, idx, Tq, topk, Hq, G, d, sm_scale, out, ws=None, ws_bytes=0,
                        stream=None):
    _check(load_library().dsa_sparse_gqa_attn(
        _ptr(q), _ptr(k), _ptr(v), dtype, n_kv, _ptr(block_table), max_blocks, block_size,
        _ptr(row_seq), _ptr(seq_lens), _ptr(idx), Tq, topk, Hq, G, d, float(sm_scale), _ptr(out),
        _ptr(ws), ws_bytes, _stream(stream)))


def dsa_prefill_workspace_size(Tq, q_pos0, chunk_rows, topk) -> int:
    return load_library().dsa_prefill_workspace_size(Tq, q_pos0, chunk_rows, topk)


def dsa_prefill(q, k, v, dtype, q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, q_pos0, Hq, G,
                d, HI, dI, topk, sm_scale, chunk_rows, out, idx_out, ws, ws_bytes, stream=None):
    _check(load_library().dsa_prefill(
        _ptr(q), _ptr(k), _ptr(v), dtype, _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx),
        _ptr(k_scale), idx_dtype, Tq, q_pos0, Hq, G, d, HI, dI, topk, float(sm_scale), chunk_rows,
        _ptr(out), _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def dsa_decode_workspace_size(B, max_blocks, block_size, topk, Hq, d) -> int:
    return load_library().dsa_decode_workspace_size(B, max_blocks, block_size, topk, Hq, d)


def dsa_prefill_stats_offset(Tq, q_pos0, chunk_rows, topk) -> int:
    return load_library().dsa_prefill_stats_offset(Tq, q_pos0, chunk_rows, topk)


def dsa_decode_stats_offset(B, max_blocks, block_size, topk, Hq, d) -> int:
    return load_library().dsa_decode_stats_offset(B, max_blocks, block_size, topk, Hq, d)


def read_stats(ws, offset, n=2):
    """The two candidate-path counters (chunks on the path, rows redone) of a workspace."""
    import torch
    if offset < 0 or offset >= (1 << 63):
        return None
    return ws.view(torch.uint8)[offset:offset + 4 * n].view(torch.int32).tolist()


def dsa_decode(q, q_idx, q_scale, w, kidx_cache, kidx_scale, k_cache, v_cache, dtype, block_table,
               seq_lens, B, num_blocks, max_blocks, block_size, Hq, G, d, HI, dI, topk, sm_scale,
               out, idx_out, ws, ws_bytes, stream=None):
    _check(load_library().dsa_decode(
        _ptr(q), _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(kidx_cache), _ptr(kidx_scale),
        _ptr(k_cache), _ptr(v_cache), dtype, _ptr(block_table), _ptr(seq_lens), B, num_blocks,
        max_blocks, block_size, Hq, G, d, HI, dI, topk, float(sm_scale), _ptr(out), _ptr(idx_out),
        _ptr(ws), ws_bytes, _stream(stream)))


def dsa_decode_noalloc_max_workspace() -> int:
    return load_library().dsa_decode_noalloc_max_workspace()


def dsa_decode_noalloc(q, q_idx, q_scale, w, kidx_cache, kidx_scale, k_cache, v_cache, dtype,
                       block_table, seq_lens, B, num_blocks, max_blocks, block_size, Hq, G, d, HI,
                       dI, topk, sm_scale, out, idx_out, stream=None):
    _check(load_library().dsa_decode_noalloc(
        _ptr(q), _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(kidx_cache), _ptr(kidx_scale),
        _ptr(k_cache), _ptr(v_cache), dtype, _ptr(block_table), _ptr(seq_lens), B, num_blocks,
        max_blocks, block_size, Hq, G, d, HI, dI, topk, float(sm_scale), _ptr(out), _ptr(idx_out),
        _stream(stream)))


# ------------------------------------------------------------ conveniences

def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def index_scores(q_idx, q_scale, w, k_idx, k_scale, q_pos0=0, stream=None):
    """Scores [Tq, ld] (fp32) of the lightning indexer; columns >= Tk are padding."""
    import torch
    Tq, HI, dI = q_idx.shape
    Tk = k_idx.shape[0]
    ld = (Tk + 3) // 4 * 4
    scores = torch.empty(Tq, ld, dtype=torch.float32, device=q_idx.device)
    n = dsa_index_scores_workspace_size(Tq, HI, dI, dtype_code(q_idx))
    ws = workspace(n, q_idx.device) if n else None
    dsa_index_scores(q_idx, q_scale, w, k_idx, k_scale, dtype_code(q_idx), Tq, Tk, HI, dI, q_pos0,
                     scores, ld, ws, n, stream)
    return scores


def topk(scores, Tk, k, q_pos0=0, stream=None):
    import torch
    Tq, ld = scores.shape
    idx = torch.empty(Tq, k, dtype=torch.int32, device=scores.device)
    n = dsa_topk_workspace_size(Tq, Tk, k)
    ws = workspace(n, scores.device) if n else None
    dsa_topk(scores, ld, Tq, Tk, q_pos0, k, idx, ws, n, stream)
    return idx


def sparse_gqa_attn(q, k, v, idx, G, sm_scale, block_table=None, block_size=0, row_seq=None,
                    seq_lens=None, split=True, stream=None):
    import torch
    Tq, Hq, d = q.shape
    topk_ = idx.shape[1]
    out = torch.empty_like(q)
    n_kv = k.shape[0]
    max_blocks = block_table.shape[1] if block_table is not None else 0
    n = dsa_sparse_gqa_attn_workspace_size(Tq, topk_, Hq, d) if split else 0
    ws = workspace(n, q.device) if n else None
    dsa_sparse_gqa_attn(q, k, v, dtype_code(q), n_kv, block_table, max_blocks, block_size, row_seq,
                        seq_lens, idx, Tq, topk_, Hq, G, d, sm_scale, out, ws, n, stream)
    return out


def _zero_stats(ws, off, n=2):
    if 0 <= off < (1 << 63):
        ws.view(__import__("torch").uint8)[off:off + 4 * n].zero_()


def dsa_sparse_gqa_attn_dedup_workspace_size(Tq, q_pos0, topk) -> int:
    return load_library().dsa_sparse_gqa_attn_dedup_workspace_size(Tq, q_pos0, topk)


def dsa_sparse_gqa_attn_dedup(q, k, v, n_kv, idx, Tq, q_pos0, topk, Hq, G, d, sm_scale, mode, out,
                              ws, ws_bytes, stream=None):
    _check(load_library().dsa_sparse_gqa_attn_dedup(
        _ptr(q), _ptr(k), _ptr(v), n_kv, _ptr(idx), Tq, q_pos0, topk, Hq, G, d, float(sm_scale),
        mode, _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_gqa_attn_dedup(q, k, v, idx, G, sm_scale, q_pos0=0, mode=0, stream=None):
    """Attention with adjacent-query deduplication (bf16, contiguous K/V); returns out."""
    import torch
    Tq, Hq, d = q.shape
    topk = idx.shape[1]
    out = torch.empty_like(q)
    n = dsa_sparse_gqa_attn_dedup_workspace_size(Tq, q_pos0, topk)
    ws = workspace(max(n, 256), q.device)
    dsa_sparse_gqa_attn_dedup(q, k, v, k.shape[0], idx, Tq, q_pos0, topk, Hq, G, d, sm_scale, mode,
                              out, ws, ws.numel(), stream)
    return out


def prefill(q, k, v, q_idx, q_scale, w, k_idx, k_scale, topk, sm_scale, chunk_rows=0, q_pos0=0,
            return_idx=False, ws=None, stream=None, return_stats=False):
    """Fused DSA prefill; returns out (and idx if return_idx, and the candidate-path
    counters [chunks on the path, rows redone] if return_stats)."""
    import torch
    Tq, Hq, d = q.shape
    G = k.shape[1]
    _, HI, dI = q_idx.shape
    out = torch.empty_like(q)
    idx = torch.empty(Tq, topk, dtype=torch.int32, device=q.device) if return_idx else None
    n = dsa_prefill_workspace_size(Tq, q_pos0, chunk_rows, topk)
    if ws is None or ws.numel() < n:
        ws = workspace(n, q.device)
    off = dsa_prefill_stats_offset(Tq, q_pos0, chunk_rows, topk) if return_stats else -1
    if return_stats:
        _zero_stats(ws, off)
    dsa_prefill(q, k, v, dtype_code(q), q_idx, q_scale, w, k_idx, k_scale, dtype_code(q_idx), Tq,
                q_pos0, Hq, G, d, HI, dI, topk, sm_scale, chunk_rows, out, idx, ws, ws.numel(),
                stream)
    res = (out, idx) if return_idx else (out,)
    if return_stats:
        res = res + (read_stats(ws, off),)
    return res if len(res) > 1 else res[0]


def decode(q, q_idx, q_scale, w, kidx_cache, kidx_scale, k_cache, v_cache, block_table, seq_lens,
           topk, sm_scale, return_idx=False, ws=None, stream=None, return_stats=False):
    """One paged DSA decode step; returns out (and idx if return_idx, and the candidate-path
    counters if return_stats: None when these shapes never take the path)."""
    import torch
    B, Hq, d = q.shape
    _, HI, dI = q_idx.shape
    NB, bs, G, _ = k_cache.shape
    max_blocks = block_table.shape[1]
    out = torch.empty_like(q)
    idx = torch.empty(B, topk, dtype=torch.int32, device=q.device) if return_idx else None
    n = dsa_decode_workspace_size(B, max_blocks, bs, topk, Hq, d)
    if ws is None or ws.numel() < n:
        ws = workspace(n, q.device)
    off = dsa_decode_stats_offset(B, max_blocks, bs, topk, Hq, d) if return_stats else -1
    if return_stats:
        _zero_stats(ws, off)
    dsa_decode(q, q_idx, q_scale, w, kidx_cache, kidx_scale, k_cache, v_cache, dtype_code(q),
               block_table, seq_lens, B, NB, max_blocks, bs, Hq, G, d, HI, dI, topk, sm_scale, out,
               idx, ws, ws.numel(), stream)
    res = (out, idx) if return_idx else (out,)
    if return_stats:
        res = res + (read_stats(ws, off),)
    return res if len(res) > 1 else res[0]


def decode_noalloc(q, q_idx, q_scale, w, kidx_cache, kidx_scale, k_cache, v_cache, block_table,
                   seq_lens, topk, sm_scale, return_idx=False, stream=None):
    """dsa_decode_noalloc: one paged DSA decode step on the library's own per-GPU scratch
    (no workspace argument); returns out (and idx if return_idx)."""
    import torch
    B, Hq, d = q.shape
    _, HI, dI = q_idx.shape
    NB, bs, G, _ = k_cache.shape
    max_blocks = block_table.shape[1]
    out = torch.empty_like(q)
    idx = torch.empty(B, topk, dtype=torch.int32, device=q.device) if return_idx else None
    dsa_decode_noalloc(q, q_idx, q_scale, w, kidx_cache, kidx_scale, k_cache, v_cache,
                       dtype_code(q), block_table, seq_lens, B, NB, max_blocks, bs, Hq, G, d, HI,
                       dI, topk, sm_scale, out, idx, stream)
    return (out, idx) if return_idx else out


def dsa_quantize_e4m3(x, x_dtype, T, n, codes, scale, stream=None):
    _check(load_library().dsa_quantize_e4m3(_ptr(x), x_dtype, T, n, _ptr(codes), _ptr(scale),
                                            _stream(stream)))


def dsa_cache_append(k_new, v_new, dtype, kidx_new, kidx_dtype, positions, block_table, B,
                     num_blocks, max_blocks, block_size, G, d, dI, k_cache, v_cache, kidx_cache,
                     kidx_scale, stream=None):
    _check(load_library().dsa_cache_append(
        _ptr(k_new), _ptr(v_new), dtype, _ptr(kidx_new), kidx_dtype, _ptr(positions),
        _ptr(block_table), B, num_blocks, max_blocks, block_size, G, d, dI, _ptr(k_cache),
        _ptr(v_cache), _ptr(kidx_cache), _ptr(kidx_scale), _stream(stream)))


def quantize_e4m3(x, stream=None):
    """Per-row E4M3 quantisation of x [..., n] (fp32 or bf16): returns (codes uint8 [..., n],
    scale float32 [...]), one scale per row of the last dimension."""
    import torch
    n = x.shape[-1]
    T = x.numel() // n if n else 0
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    dsa_quantize_e4m3(x, dtype_code(x), T, n, codes, scale, stream)
    return codes, scale


def cache_append(k_new, v_new, kidx_new, positions, block_table, k_cache, v_cache, kidx_cache,
                 kidx_scale, stream=None):
    """Write one token per sequence (k_new / v_new [B, G, d], kidx_new [B, dI]) into the paged
    caches in place, at positions [B] (int32, device) through block_table [B, max_blocks]."""
    B, G, d = k_new.shape
    NB, bs = k_cache.shape[:2]
    dsa_cache_append(k_new, v_new, dtype_code(k_new), kidx_new, dtype_code(kidx_new), positions,
                     block_table, B, NB, block_table.shape[1], bs, G, d, kidx_new.shape[-1],
                     k_cache, v_cache, kidx_cache, kidx_scale, stream)


def dsa_prefill_varlen(q, k, v, dtype, q_idx, q_scale, w, k_idx, k_scale, idx_dtype, cu_seqlens,
                       nseq, Hq, G, d, HI, dI, topk, sm_scale, chunk_rows, out, idx_out=None,
                       ws=None, ws_bytes=0, stream=None):
    """cu_seqlens: a host sequence of nseq + 1 ints (list, numpy array or CPU tensor)."""
    cu = (ctypes.c_int32 * (nseq + 1))(*[int(c) for c in list(cu_seqlens)[:nseq + 1]])
    _check(load_library().dsa_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), dtype, _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx),
        _ptr(k_scale), idx_dtype, ctypes.cast(cu, ctypes.c_void_p), nseq, Hq, G, d, HI, dI, topk,
        float(sm_scale), chunk_rows, _ptr(out), _ptr(idx_out), _ptr(ws), ws_bytes,
        _stream(stream)))


def prefill_varlen(q, k, v, q_idx, q_scale, w, k_idx, k_scale, cu_seqlens, topk, sm_scale,
                   chunk_rows=0, return_idx=False, ws=None, stream=None, return_stats=False):
    """Packed variable-length prefill: sequence i is tokens cu_seqlens[i] .. cu_seqlens[i+1]-1
    of every array.  Returns out (and idx with positions local to each sequence, and the
    candidate-path counters, as for ``prefill``)."""
    import torch
    cu = [int(c) for c in list(cu_seqlens)]
    nseq = len(cu) - 1
    T, Hq, d = q.shape
    G = k.shape[1]
    _, HI, dI = q_idx.shape
    out = torch.empty_like(q)
    idx = torch.empty(T, topk, dtype=torch.int32, device=q.device) if return_idx else None
    max_len = max([b - a for a, b in zip(cu[:-1], cu[1:])] + [0])
    n = dsa_prefill_workspace_size(max_len, 0, chunk_rows, topk) if max_len > 0 else 0
    if ws is None or ws.numel() < n:
        ws = workspace(max(n, 256), q.device)
    off = dsa_prefill_stats_offset(max_len, 0, chunk_rows, topk) if return_stats and max_len else -1
    if return_stats:
        _zero_stats(ws, off)
    dsa_prefill_varlen(q, k, v, dtype_code(q), q_idx, q_scale, w, k_idx, k_scale,
                       dtype_code(q_idx), cu, nseq, Hq, G, d, HI, dI, topk, sm_scale, chunk_rows,
                       out, idx, ws, ws.numel(), stream)
    res = (out, idx) if return_idx else (out,)
    if return_stats:
        res = res + (read_stats(ws, off) if off >= 0 else [0, 0],)
    return res if len(res) > 1 else res[0]


# ------------------------------------------------------------------ training side

def dsa_index_scores_at(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI, idx, topk,
                        vals, stream=None):
    _check(load_library().dsa_index_scores_at(
        _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale), idx_dtype, Tq, Tk, HI,
        dI, _ptr(idx), topk, _ptr(vals), _stream(stream)))


def dsa_index_scores_at_bwd_workspace_size(Tq, Tk, HI, topk) -> int:
    return load_library().dsa_index_scores_at_bwd_workspace_size(Tq, Tk, HI, topk)


def dsa_index_scores_at_bwd(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI, idx,
                            topk, g, dq_idx, dw, dk_idx, ws=None, ws_bytes=0, stream=None):
    _check(load_library().dsa_index_scores_at_bwd(
        _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale), idx_dtype, Tq, Tk, HI,
        dI, _ptr(idx), topk, _ptr(g), _ptr(dq_idx), _ptr(dw), _ptr(dk_idx), _ptr(ws), ws_bytes,
        _stream(stream)))


def index_scores_at(q_idx, q_scale, w, k_idx, k_scale, idx, stream=None):
    """I[t, idx[t, i]] (fp32 [Tq, topk], -inf for padding) of FP8 indexer inputs."""
    import torch
    Tq, HI, dI = q_idx.shape
    vals = torch.empty(idx.shape, dtype=torch.float32, device=q_idx.device)
    dsa_index_scores_at(q_idx, q_scale, w, k_idx, k_scale, DSA_FP8_E4M3, Tq, k_idx.shape[0], HI,
                        dI, idx, idx.shape[1], vals, stream)
    return vals


def index_scores_at_bwd(q_idx, q_scale, w, k_idx, k_scale, idx, g, staged=True, ws=None,
                        stream=None):
    """(dq_idx [Tq, HI, dI], dw [Tq, HI], dk_idx [Tk, dI]) fp32 gradients of sum g * vals;
    staged: the deterministic reduction of dk_idx through a workspace when H^I allows it."""
    import torch
    Tq, HI, dI = q_idx.shape
    dq = torch.empty(Tq, HI, dI, dtype=torch.float32, device=q_idx.device)
    dw = torch.empty(Tq, HI, dtype=torch.float32, device=q_idx.device)
    dk = torch.zeros(k_idx.shape[0], dI, dtype=torch.float32, device=q_idx.device)
    n = dsa_index_scores_at_bwd_workspace_size(Tq, k_idx.shape[0], HI, idx.shape[1]) if staged else 0
    if n and (ws is None or ws.numel() < n):
        ws = workspace(n, q_idx.device)
    dsa_index_scores_at_bwd(q_idx, q_scale, w, k_idx, k_scale, DSA_FP8_E4M3, Tq, k_idx.shape[0],
                            HI, dI, idx, idx.shape[1], g, dq, dw, dk, ws if n else None,
                            ws.numel() if n else 0, stream)
    return dq, dw, dk


def dsa_sparse_gqa_attn_lse(q, k, v, dtype, n_kv, idx, Tq, topk, Hq, G, d, sm_scale, out, lse,
                            ws=None, ws_bytes=0, stream=None):
    _check(load_library().dsa_sparse_gqa_attn_lse(
        _ptr(q), _ptr(k), _ptr(v), dtype, n_kv, _ptr(idx), Tq, topk, Hq, G, d, float(sm_scale),
        _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def dsa_sparse_gqa_attn_bwd_workspace_size(Tq, topk, G, n_kv) -> int:
    return load_library().dsa_sparse_gqa_attn_bwd_workspace_size(Tq, topk, G, n_kv)


def dsa_sparse_gqa_attn_bwd(q, k, v, dtype, n_kv, idx, Tq, topk, Hq, G, d, sm_scale, out, dout,
                            lse, dq, dk, dv, vals=None, kl=None, dI=None, ws=None, ws_bytes=0,
                            stream=None):
    _check(load_library().dsa_sparse_gqa_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), dtype, n_kv, _ptr(idx), Tq, topk, Hq, G, d, float(sm_scale),
        _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(vals), _ptr(kl),
        _ptr(dI), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_gqa_attn_lse(q, k, v, idx, G, sm_scale, stream=None):
    """(out, lse fp32 [Tq, Hq]) of the attention over contiguous K/V."""
    import torch
    Tq, Hq, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty(Tq, Hq, dtype=torch.float32, device=q.device)
    n = dsa_sparse_gqa_attn_workspace_size(Tq, idx.shape[1], Hq, d)
    ws = workspace(n, q.device) if n else None
    dsa_sparse_gqa_attn_lse(q, k, v, dtype_code(q), k.shape[0], idx, Tq, idx.shape[1], Hq, G, d,
                            sm_scale, out, lse, ws, n, stream)
    return out, lse


def sparse_gqa_attn_bwd(q, k, v, idx, G, sm_scale, out, dout, lse, vals=None, staged=True,
                        ws=None, stream=None):
    """(dq bf16, dk fp32, dv fp32[, kl, dI]) of the attention (and the sparse indexer loss when
    vals, the indexer scores at idx, is given).  staged: the deterministic reduction of dK / dV
    through a workspace (else fp32 atomic adds)."""
    import torch
    Tq, Hq, d = q.shape
    dq = torch.empty_like(q)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=q.device)
    kl = dI = None
    if vals is not None:
        kl = torch.empty(Tq, dtype=torch.float32, device=q.device)
        dI = torch.empty(idx.shape, dtype=torch.float32, device=q.device)
    n = dsa_sparse_gqa_attn_bwd_workspace_size(Tq, idx.shape[1], G, k.shape[0]) if staged else 0
    if n and (ws is None or ws.numel() < n):
        ws = workspace(n, q.device)
    dsa_sparse_gqa_attn_bwd(q, k, v, dtype_code(q), k.shape[0], idx, Tq, idx.shape[1], Hq, G, d,
                            sm_scale, out, dout, lse, dq, dk, dv, vals, kl, dI,
                            ws if n else None, ws.numel() if n else 0, stream)
    return (dq, dk, dv) if vals is None else (dq, dk, dv, kl, dI)


def dsa_indexer_warmup_kl(q, k, dtype, Tq, Tk, q_pos0, Hq, G, d, sm_scale, lse, scores, ld_scores,
                          kl, stream=None):
    _check(load_library().dsa_indexer_warmup_kl(
        _ptr(q), _ptr(k), dtype, Tq, Tk, q_pos0, Hq, G, d, float(sm_scale), _ptr(lse),
        _ptr(scores), ld_scores, _ptr(kl), _stream(stream)))


def dsa_index_scores_bwd_dense_workspace_size(Tq, Tk, HI) -> int:
    return load_library().dsa_index_scores_bwd_dense_workspace_size(Tq, Tk, HI)


def dsa_index_scores_bwd_dense(q_idx, q_scale, w, k_idx, k_scale, idx_dtype, Tq, Tk, HI, dI,
                               q_pos0, g, ld_g, dq_idx, dw, dk_idx, ws=None, ws_bytes=0,
                               stream=None):
    _check(load_library().dsa_index_scores_bwd_dense(
        _ptr(q_idx), _ptr(q_scale), _ptr(w), _ptr(k_idx), _ptr(k_scale), idx_dtype, Tq, Tk, HI, dI,
        q_pos0, _ptr(g), ld_g, _ptr(dq_idx), _ptr(dw), _ptr(dk_idx), _ptr(ws), ws_bytes,
        _stream(stream)))


def indexer_warmup_kl(q, k, G, sm_scale, scores, Tk, q_pos0=0, lse=None, stream=None):
    """Dense warm-up loss: kl [Tq] fp32; scores [Tq, ld] (I over the causal prefix) is
    overwritten in place with dL/dI."""
    import torch
    Tq, Hq, d = q.shape
    kl = torch.empty(Tq, dtype=torch.float32, device=q.device)
    dsa_indexer_warmup_kl(q, k, dtype_code(q), Tq, Tk, q_pos0, Hq, G, d, sm_scale, lse, scores,
                          scores.shape[1], kl, stream)
    return kl


def index_scores_bwd_dense(q_idx, q_scale, w, k_idx, k_scale, g, Tk, q_pos0=0, dk=None, ws=None,
                           stream=None):
    """(dq_idx [Tq, HI, dI], dw [Tq, HI], dk_idx [Tk, dI]) fp32 gradients of
    sum_{s <= pos} g[t, s] I[t, s]; dk (if given) is accumulated into."""
    import torch
    Tq, HI, dI = q_idx.shape
    dq = torch.empty(Tq, HI, dI, dtype=torch.float32, device=q_idx.device)
    dw = torch.empty(Tq, HI, dtype=torch.float32, device=q_idx.device)
    if dk is None:
        dk = torch.zeros(Tk, dI, dtype=torch.float32, device=q_idx.device)
    n = dsa_index_scores_bwd_dense_workspace_size(Tq, Tk, HI)
    if n and (ws is None or ws.numel() < n):
        ws = workspace(n, q_idx.device)
    dsa_index_scores_bwd_dense(q_idx, q_scale, w, k_idx, k_scale, DSA_FP8_E4M3, Tq, Tk, HI, dI,
                               q_pos0, g, g.shape[1], dq, dw, dk, ws if n else None,
                               ws.numel() if n else 0, stream)
    return dq, dw, dk
