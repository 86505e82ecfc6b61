"""The C-ABI boundary on the host: exports, workspace sizing and argument checks.

No kernel runs here: every call below fails validation, which happens on the
host before anything is queued (fake, never-dereferenced device addresses).
"""
import ctypes
import os
import re

import pytest

import long_context_sparse_02_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
A = 0x10000          # a 16-byte aligned fake device address
MIS = 0x10004        # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dsa.LIB_PATH):
        from long_context_sparse_02_amd import build
        build.build()
    return dsa.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(dsa.EXPORTS)


def test_status_strings_and_version(lib):
    for code, name in dsa.STATUS.items():
        assert lib.dsa_status_string(code).decode() == name
    assert lib.dsa_version() >= 10000


def _st(lib, fn, *args):
    return getattr(lib, fn)(*args)


def test_index_scores_argument_checks(lib):
    f = lib.dsa_index_scores
    ok = [A, A, A, A, A, dsa.DSA_FP8_E4M3, 16, 16, 64, 128, 0, A, 16, A, 1 << 20, None]
    assert f(*ok[:0], None, *ok[1:]) == 1                      # NULL q_idx
    assert b"q_idx" in lib.dsa_last_error()
    bad = list(ok); bad[0] = MIS
    assert f(*bad) == 1 and b"aligned" in lib.dsa_last_error()
    bad = list(ok); bad[9] = 64
    assert f(*bad) == 2                                         # FP8 needs dI = 128
    bad = list(ok); bad[8] = 6
    assert f(*bad) == 2                                         # HI % 4
    bad = list(ok); bad[7] = 15
    assert f(*bad) == 1                                         # Tk < q_pos0 + Tq
    bad = list(ok); bad[10] = 3
    assert f(*bad) == 1
    bad = list(ok); bad[12] = 14
    assert f(*bad) == 1                                         # ld < Tk
    bad = list(ok); bad[12] = 18
    assert f(*bad) == 1                                         # ld % 4
    bad = list(ok); bad[5] = dsa.DSA_BF16
    assert f(*bad) == 2                                         # bf16 indexer unsupported
    bad = list(ok); bad[1] = None
    assert f(*bad) == 1                                         # FP8 needs scales
    bad = list(ok); bad[5] = dsa.DSA_F32; bad[9] = 64; bad[8] = 32
    assert f(*bad) == 2                                         # fp32: HI * dI > 1024
    n = lib.dsa_index_scores_workspace_size(16, 64, 128, dsa.DSA_FP8_E4M3)
    assert n >= 16 * 512
    assert lib.dsa_index_scores_workspace_size(16, 8, 64, dsa.DSA_F32) == 0
    bad = list(ok); bad[14] = n - 1
    assert f(*bad) == 3                                         # FP8 indexer scratch too small
    bad = list(ok); bad[13] = None
    assert f(*bad) == 3


def test_topk_argument_checks(lib):
    f = lib.dsa_topk
    ok = [A, 16, 8, 16, 8, 4, A, None, 0, None]
    bad = list(ok); bad[5] = 0
    assert f(*bad) == 1
    bad = list(ok); bad[5] = 8193
    assert f(*bad) == 1
    bad = list(ok); bad[3] = 15
    assert f(*bad) == 1
    bad = list(ok); bad[6] = None
    assert f(*bad) == 1
    bad = list(ok); bad[1] = 17
    assert f(*bad) == 1
    assert lib.dsa_topk_workspace_size(8192, 131072, 2048) == 0   # many rows: one pass each
    assert lib.dsa_topk_workspace_size(64, 262144, 2048) >= 64 * 4 * 2048 * 4   # few long rows: split


def test_attention_argument_checks(lib):
    f = lib.dsa_sparse_gqa_attn
    ok = [A, A, A, dsa.DSA_BF16, 100, None, 0, 0, None, None, A, 4, 16, 32, 4, 128, 0.1, A, None, 0, None]
    bad = list(ok); bad[15] = 64
    assert f(*bad) == 2                                         # d != 128
    bad = list(ok); bad[13] = 30
    assert f(*bad) == 1                                         # Hq % G
    bad = list(ok); bad[13] = 68
    assert f(*bad) == 2                                         # > 16 heads per group
    bad = list(ok); bad[3] = dsa.DSA_FP8_E4M3
    assert f(*bad) == 2
    bad = list(ok); bad[12] = 0
    assert f(*bad) == 1
    bad = list(ok); bad[5] = A; bad[6] = 0
    assert f(*bad) == 1                                         # paged without max_blocks
    bad = list(ok); bad[17] = MIS
    assert f(*bad) == 1


def test_prefill_and_decode_workspace_checks(lib):
    n = lib.dsa_prefill_workspace_size(1000, 0, 256, 64)
    assert n >= 256 * 1000 * 4 + 256 * 64 * 4
    assert lib.dsa_prefill_workspace_size(1000, 0, 0, 64) >= 1000 * 1000 * 4
    f = lib.dsa_prefill
    args = [A, A, A, dsa.DSA_BF16, A, A, A, A, A, dsa.DSA_FP8_E4M3, 1000, 0, 32, 4, 128, 64, 128,
            64, 0.1, 256, A, None, A, n - 1, None]
    assert f(*args) == 3 and b"workspace" in lib.dsa_last_error()
    args[22] = None
    assert f(*args) == 3
    nd = lib.dsa_decode_workspace_size(64, 4096, 64, 2048, 32, 128)
    assert nd >= 64 * 4096 * 64 * 4
    fd = lib.dsa_decode
    dargs = [A, A, A, A, A, A, A, A, dsa.DSA_BF16, A, A, 64, 1000, 4096, 64, 32, 4, 128, 64, 128,
             2048, 0.1, A, None, A, nd - 16, None]
    assert fd(*dargs) == 3
    dargs[19] = 64
    assert fd(*dargs) == 2                                      # decode dI must be 128
    dargs[19] = 128; dargs[14] = 16
    assert fd(*dargs) == 2                                      # 64-token blocks only
    dargs[14] = 64; dargs[10] = None
    assert fd(*dargs) == 1                                      # seq_lens NULL


def test_decode_noalloc_checks(lib):
    """The no-allocation decode step: its scratch limit, and the checks it shares with
    dsa_decode (all on the host, before any device call)."""
    cap = lib.dsa_decode_noalloc_max_workspace()
    assert cap == 96 << 20
    # the 64-sequence step over 256K-token caches fits
    assert lib.dsa_decode_workspace_size(64, 4096, 64, 2048, 32, 128) <= cap
    f = lib.dsa_decode_noalloc
    dargs = [A, A, A, A, A, A, A, A, dsa.DSA_BF16, A, A, 128, 1000, 4096, 64, 32, 4, 128, 64, 128,
             2048, 0.1, A, None, None]
    assert lib.dsa_decode_workspace_size(128, 4096, 64, 2048, 32, 128) > cap
    assert f(*dargs) == 3                                       # beyond the scratch
    assert b"dsa_decode_noalloc" in lib.dsa_last_error()
    dargs[11] = 64
    dargs[19] = 64
    assert f(*dargs) == 2                                       # dI must be 128
    dargs[19] = 128; dargs[14] = 16
    assert f(*dargs) == 2                                       # 64-token blocks only
    dargs[14] = 64; dargs[10] = None
    assert f(*dargs) == 1                                       # seq_lens NULL
    dargs[10] = A; dargs[22] = MIS
    assert f(*dargs) == 1                                       # out misaligned
    dargs[22] = A; dargs[11] = -1
    assert f(*dargs) == 1                                       # negative batch
    dargs[11] = 0
    assert f(*dargs) == 0                                       # empty batch: nothing to do


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        dsa._ptr(x)


def test_quantize_and_cache_append_argument_checks(lib):
    q = lib.dsa_quantize_e4m3
    assert q(A, dsa.DSA_F32, 0, 128, None, None, None) == 0           # nothing to do
    assert q(A, dsa.DSA_FP8_E4M3, 4, 128, A, A, None) == 2             # input must be f32/bf16
    assert q(None, dsa.DSA_F32, 4, 128, A, A, None) == 1 and b"x" in lib.dsa_last_error()
    assert q(A, dsa.DSA_BF16, 4, 128, A, 0x10002, None) == 1           # scale misaligned
    assert q(A, dsa.DSA_F32, -1, 128, A, A, None) == 1
    assert q(A, dsa.DSA_F32, 4, 0, A, A, None) == 1
    c = lib.dsa_cache_append
    ok = [A, A, dsa.DSA_BF16, A, dsa.DSA_F32, A, A, 8, 100, 64, 64, 4, 128, 128, A, A, A, A, None]
    bad = list(ok); bad[7] = 0
    assert c(*bad) == 0                                                # B = 0: nothing queued
    bad = list(ok); bad[0] = MIS
    assert c(*bad) == 1 and b"k_new" in lib.dsa_last_error()
    bad = list(ok); bad[2] = dsa.DSA_FP8_E4M3
    assert c(*bad) == 2
    bad = list(ok); bad[4] = dsa.DSA_FP8_E4M3
    assert c(*bad) == 2
    bad = list(ok); bad[11], bad[12] = 1, 4                            # 8-byte K/V rows
    assert c(*bad) == 2 and b"16 bytes" in lib.dsa_last_error()
    bad = list(ok); bad[5] = None
    assert c(*bad) == 1 and b"positions" in lib.dsa_last_error()
    bad = list(ok); bad[16] = None
    assert c(*bad) == 1 and b"kidx_cache" in lib.dsa_last_error()
    bad = list(ok); bad[10] = 0
    assert c(*bad) == 1


def test_prefill_varlen_argument_checks(lib):
    f = lib.dsa_prefill_varlen

    def cu(*v):
        return ctypes.cast((ctypes.c_int32 * len(v))(*v), ctypes.c_void_p)
    n = lib.dsa_prefill_workspace_size(3000, 0, 1024, 2048)
    args = [A, A, A, dsa.DSA_BF16, A, A, A, A, A, dsa.DSA_FP8_E4M3, cu(0, 1000, 1000, 4000), 3,
            32, 4, 128, 64, 128, 2048, 0.1, 1024, A, None, A, n - 1, None]
    assert f(*args) == 3 and b"workspace" in lib.dsa_last_error()   # sized by the longest
    args[10] = None
    assert f(*args) == 1 and b"cu_seqlens" in lib.dsa_last_error()
    args[10] = cu(1, 1000)
    args[11] = 1
    assert f(*args) == 1 and b"cu_seqlens[0]" in lib.dsa_last_error()
    args[10] = cu(0, 1000, 999)
    args[11] = 2
    assert f(*args) == 1 and b"decrease" in lib.dsa_last_error()
    args[10] = cu(0, 0, 0)
    assert f(*args) == 0                                             # only empty sequences
    args[10] = cu(0, 100)
    args[11] = 1
    args[15] = 6
    assert f(*args) == 2                                             # FP8 needs HI % 4 == 0


def test_training_side_argument_checks(lib):
    f = lib.dsa_index_scores_at
    ok = [A, A, A, A, A, dsa.DSA_FP8_E4M3, 16, 100, 64, 128, A, 2048, A, None]
    bad = list(ok); bad[5] = dsa.DSA_F32
    assert f(*bad) == 2                                          # FP8 only
    bad = list(ok); bad[9] = 64
    assert f(*bad) == 2                                          # dI must be 128
    bad = list(ok); bad[12] = None
    assert f(*bad) == 1 and b"vals" in lib.dsa_last_error()
    fb = lib.dsa_index_scores_at_bwd
    okb = [A, A, A, A, A, dsa.DSA_FP8_E4M3, 16, 100, 64, 128, A, 2048, A, A, A, A, None, 0, None]
    bad = list(okb); bad[8] = 128
    assert fb(*bad) == 2                                         # the backward takes HI <= 64
    bad = list(okb); bad[15] = None
    assert fb(*bad) == 1 and b"dk_idx" in lib.dsa_last_error()
    assert lib.dsa_index_scores_at_bwd_workspace_size(16, 100, 12, 2048) == 0   # no staged form
    n = lib.dsa_index_scores_at_bwd_workspace_size(16, 100, 64, 2048)
    assert n >= 32 * 2048 * 512
    bad = list(okb); bad[16] = A; bad[17] = n - 1
    assert fb(*bad) == 3 and b"workspace" in lib.dsa_last_error()
    bad = list(okb); bad[8] = 12; bad[16] = A; bad[17] = n
    assert fb(*bad) == 2 and b"multiple of 16" in lib.dsa_last_error()
    fl = lib.dsa_sparse_gqa_attn_lse
    okl = [A, A, A, dsa.DSA_BF16, 100, A, 16, 2048, 32, 4, 128, 0.1, A, A, None, 0, None]
    bad = list(okl); bad[13] = None
    assert fl(*bad) == 1 and b"lse" in lib.dsa_last_error()
    bad = list(okl); bad[10] = 64
    assert fl(*bad) == 2
    fw = lib.dsa_sparse_gqa_attn_bwd
    okw = [A, A, A, dsa.DSA_BF16, 100, A, 16, 2048, 32, 4, 128, 0.1, A, A, A, A, A, A, A, A, A,
           None, 0, None]
    bad = list(okw); bad[3] = dsa.DSA_F32
    assert fw(*bad) == 2 and b"BF16" in lib.dsa_last_error()
    bad = list(okw); bad[7] = 4096
    assert fw(*bad) == 2 and b"2048" in lib.dsa_last_error()  # the fused loss: topk <= 2048
    bad = list(okw); bad[20] = None
    assert fw(*bad) == 1 and b"dI" in lib.dsa_last_error()
    bad = list(okw); bad[14] = None
    assert fw(*bad) == 1 and b"lse" in lib.dsa_last_error()
    n = lib.dsa_sparse_gqa_attn_bwd_workspace_size(16, 2048, 4, 100)
    assert n >= 32 * 2048 * 4 * 1024                            # a chunk of staged contributions
    bad = list(okw); bad[21] = A; bad[22] = n - 1
    assert fw(*bad) == 3 and b"workspace" in lib.dsa_last_error()
    bad = list(okw); bad[22] = 64                                # size without a buffer
    assert fw(*bad) == 3


def test_warmup_argument_checks(lib):
    """Every call below carries one bad argument, so validation fails before any launch."""
    f = lib.dsa_indexer_warmup_kl
    ok = [A, A, dsa.DSA_BF16, 16, 100, 84, 32, 4, 128, 0.1, None, A, 100, A, None]
    bad = list(ok); bad[2] = dsa.DSA_F32
    assert f(*bad) == 2 and b"BF16" in lib.dsa_last_error()
    bad = list(ok); bad[8] = 64
    assert f(*bad) == 2                                          # d must be 128
    bad = list(ok); bad[6] = 48; bad[7] = 8                      # 6 heads per group
    assert f(*bad) == 2
    bad = list(ok); bad[6] = 128; bad[7] = 4                     # 4 groups x 8 waves each
    assert f(*bad) == 2
    bad = list(ok); bad[5] = 85                                  # last row's prefix beyond Tk
    assert f(*bad) == 1 and b"prefix" in lib.dsa_last_error()
    bad = list(ok); bad[12] = 99
    assert f(*bad) == 1 and b"ld_scores" in lib.dsa_last_error()
    bad = list(ok); bad[13] = None
    assert f(*bad) == 1 and b"kl" in lib.dsa_last_error()
    bad = list(ok); bad[10] = A + 2; bad[13] = None              # misaligned lse caught first
    assert f(*bad) == 1 and b"lse" in lib.dsa_last_error()
    fb = lib.dsa_index_scores_bwd_dense
    okb = [A, A, A, A, A, dsa.DSA_FP8_E4M3, 16, 100, 64, 128, 84, A, 100, A, A, A, None, 0, None]
    bad = list(okb); bad[5] = dsa.DSA_F32
    assert fb(*bad) == 2
    bad = list(okb); bad[8] = 12
    assert fb(*bad) == 2 and b"HI" in lib.dsa_last_error()
    bad = list(okb); bad[8] = 128
    assert fb(*bad) == 2
    bad = list(okb); bad[10] = 90
    assert fb(*bad) == 1 and b"prefix" in lib.dsa_last_error()
    bad = list(okb); bad[15] = None
    assert fb(*bad) == 1 and b"dk_idx" in lib.dsa_last_error()
    assert lib.dsa_index_scores_bwd_dense_workspace_size(16, 100, 12) == 0
    n = lib.dsa_index_scores_bwd_dense_workspace_size(16, 100, 64)
    assert n >= 16 * 128 * 64 * 2 + 128 * 128 * 2               # bf16 copies of the codes
    bad = list(okb)                                              # no workspace
    assert fb(*bad) == 3 and b"workspace" in lib.dsa_last_error()
    bad = list(okb); bad[16] = A; bad[17] = n - 1
    assert fb(*bad) == 3
