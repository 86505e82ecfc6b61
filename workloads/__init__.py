"""Seeded synthetic inputs for the DSA layer.

This module only draws random numbers and lays them out; it holds none of
the layer's arithmetic.  Both the GPU library and the CPU oracle consume the
exact bytes it produces.

Shapes follow the attention geometry of a Qwen3-30B-A3B-style backbone as the
Keye-VL-2.0 report uses it (32 query heads, 4 KV groups, head size 128) with
an MQA-style FP8 lightning indexer (64 indexer heads of size 128) and k = 2048
(report section 2.3; xllm-io review page, "核心公式").  The pages measure real
video contexts on the trained model; those activations and weights are not
available, so these generators stand in for them:

  * q, k, v ~ N(0, 1) / sqrt(d) (bf16, or fp32 for the tiny case);
  * indexer queries q^I ~ N(0, 1); gate weights w ~ U(0, 1);
  * indexer keys k^I ~ N(0, 1), or clustered: one Gaussian centre per frame
    span plus 0.3 * N(0, 1) noise (report section 2.3: long video contexts;
    15-second clips interleaved with text, report section 3);
  * FP8 indexer tensors are per-token scaled E4M3 codes: scale = amax / 448
    over the token's values (1 if all are zero), codes = RNE(x / scale)
    after clamping to +-448.

Generation runs on whatever torch device is given (the GPU for the large
workloads; the bytes are copied to the host for the oracle).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    L: int                 # sequence length (queries = keys = L)
    HI: int = 64           # indexer heads
    dI: int = 128          # indexer head size
    idx_dtype: str = "fp8"  # "fp8" or "f32"
    k: int = 2048          # top-k budget
    Hq: int = 32           # query heads
    G: int = 4             # KV groups
    d: int = 128           # head size
    dtype: str = "bf16"    # "bf16" or "f32"
    chunk: int = 0         # query rows per chunk (0 = one chunk)
    keys: str = "iid"      # "iid", "clustered" or "multimodal"
    cluster_span: int = 256
    cluster_std: float = 0.3
    vision_tokens: int = 3840   # multimodal: vision tokens per 15 s segment
    text_tokens: int = 128      # multimodal: text tokens per segment
    queries: str = "iid"        # indexer queries: "iid", or "frames" (a centre per frame span)
    query_std: float = 0.5      # "frames": noise around a query's frame centre
    seed: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int = 64
    Lmin: int = 32768
    Lmax: int = 262144
    block: int = 64
    HI: int = 64
    dI: int = 128
    k: int = 2048
    Hq: int = 32
    G: int = 4
    d: int = 128
    dtype: str = "bf16"
    seed: int = 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads: a tiny fp32 layer, 32K / 128K / 256K prefill and paged
# decode, plus the 256K point of the decode curve.
TINY_F32 = PrefillConfig("tiny_f32_2k", L=2048, HI=8, dI=64, idx_dtype="f32", k=256, Hq=8,
                         G=2, d=128, dtype="f32", seed=1001)
PREFILL_32K = PrefillConfig("prefill_32k", L=32768, seed=1002)
PREFILL_128K = PrefillConfig("prefill_128k_clustered", L=131072, chunk=8192, keys="clustered",
                             seed=1003)
DECODE_PAGED = DecodeConfig("decode_paged_64x32k-256k", seed=1004)
PREFILL_256K_MM = PrefillConfig("prefill_256k_multimodal", L=262144, chunk=16384,
                                keys="multimodal", seed=1005)
DECODE_256K = DecodeConfig("decode_paged_64x256k", Lmin=262144, Lmax=262144, seed=1006)

ALL = {c.name: c for c in (TINY_F32, PREFILL_32K, PREFILL_128K, DECODE_PAGED, PREFILL_256K_MM,
                           DECODE_256K)}


def _gen(seed: int, tensor_id: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + tensor_id)
    return g


def quantize_e4m3_per_token(x: torch.Tensor):
    """Per-token (first dimension) scaled OCP E4M3 codes.  Returns (uint8 codes, fp32 scales)."""
    T = x.shape[0]
    flat = x.reshape(T, -1).float()
    amax = flat.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (flat / scale[:, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return codes.view(torch.uint8).reshape(x.shape).contiguous(), scale.contiguous()


def _indexer_keys(cfg: PrefillConfig, device) -> torch.Tensor:
    L, dI = cfg.L, cfg.dI
    g = _gen(cfg.seed, 5, device)
    if cfg.keys == "iid":
        return torch.randn(L, dI, generator=g, device=device)
    noise = torch.randn(L, dI, generator=g, device=device)
    gc = _gen(cfg.seed, 6, device)
    if cfg.keys == "clustered":
        n_clusters = (L + cfg.cluster_span - 1) // cfg.cluster_span
        centres = torch.randn(n_clusters, dI, generator=gc, device=device)
        cid = torch.arange(L, device=device) // cfg.cluster_span
        return centres[cid] + cfg.cluster_std * noise
    if cfg.keys == "multimodal":
        seg = cfg.vision_tokens + cfg.text_tokens
        pos = torch.arange(L, device=device)
        in_seg = pos % seg
        is_vision = in_seg < cfg.vision_tokens
        frames_per_seg = cfg.vision_tokens // cfg.cluster_span
        frame = (pos // seg) * frames_per_seg + in_seg // cfg.cluster_span
        n_frames = int(frame.max().item()) + 1
        centres = torch.randn(n_frames, dI, generator=gc, device=device)
        vision = centres[frame.clamp(max=n_frames - 1)] + cfg.cluster_std * noise
        return torch.where(is_vision[:, None], vision, noise)
    raise ValueError(cfg.keys)


def _indexer_queries(cfg: PrefillConfig, device) -> torch.Tensor:
    """q^I [L, HI, dI]: i.i.d. N(0, 1), or with frame structure: the tokens of one frame span
    (cluster_span tokens; in the multimodal layout the vision tokens of one frame) share a
    per-head N(0, I) centre and add query_std * N(0, 1); multimodal text tokens stay i.i.d.
    Adjacent queries of one frame then pick mostly the same keys, as video tokens of one frame
    do (report section 5.3: 16 adjacent queries need about 8K distinct keys at 128K)."""
    L, HI, dI = cfg.L, cfg.HI, cfg.dI
    noise = torch.randn(L, HI, dI, generator=_gen(cfg.seed, 4, device), device=device)
    if cfg.queries == "iid":
        return noise
    if cfg.queries != "frames":
        raise ValueError(cfg.queries)
    pos = torch.arange(L, device=device)
    if cfg.keys == "multimodal":
        seg = cfg.vision_tokens + cfg.text_tokens
        in_seg = pos % seg
        frame = (pos // seg) * (cfg.vision_tokens // cfg.cluster_span) + in_seg // cfg.cluster_span
        text = in_seg >= cfg.vision_tokens
    else:
        frame = pos // cfg.cluster_span
        text = torch.zeros(L, dtype=torch.bool, device=device)
    n_frames = int(frame.max().item()) + 1
    centres = torch.randn(n_frames, HI, dI, generator=_gen(cfg.seed, 8, device), device=device)
    q = centres[frame] + cfg.query_std * noise
    return torch.where(text[:, None, None], noise, q)


def prefill_inputs(cfg: PrefillConfig, device="cpu") -> dict:
    """All inputs of one prefill layer call, on ``device``."""
    L = cfg.L
    el = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    s = 1.0 / math.sqrt(cfg.d)
    out = {}
    out["q"] = (torch.randn(L, cfg.Hq, cfg.d, generator=_gen(cfg.seed, 1, device), device=device) * s).to(el)
    out["k"] = (torch.randn(L, cfg.G, cfg.d, generator=_gen(cfg.seed, 2, device), device=device) * s).to(el)
    out["v"] = (torch.randn(L, cfg.G, cfg.d, generator=_gen(cfg.seed, 3, device), device=device) * s).to(el)
    qi = _indexer_queries(cfg, device)
    ki = _indexer_keys(cfg, device)
    out["w"] = torch.rand(L, cfg.HI, generator=_gen(cfg.seed, 7, device), device=device)
    if cfg.idx_dtype == "fp8":
        out["q_idx"], out["q_scale"] = quantize_e4m3_per_token(qi)
        out["k_idx"], out["k_scale"] = quantize_e4m3_per_token(ki)
    else:
        out["q_idx"], out["q_scale"] = qi.contiguous(), None
        out["k_idx"], out["k_scale"] = ki.contiguous(), None
    del qi, ki
    return out


def decode_inputs(cfg: DecodeConfig, device="cpu", lens: Optional[torch.Tensor] = None) -> dict:
    """One paged decode step: B sequences, each with its own last token as the query.

    The caches hold every sequence's tokens in blocks of ``cfg.block`` tokens
    whose physical order is a seeded permutation.
    """
    B, bs = cfg.B, cfg.block
    el = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    s = 1.0 / math.sqrt(cfg.d)
    if lens is None:
        lens = torch.randint(cfg.Lmin, cfg.Lmax + 1, (B,), generator=_gen(cfg.seed, 10, "cpu"))
    lens = lens.to(torch.int32).cpu()
    nblk = (lens + bs - 1) // bs
    NB = int(nblk.sum().item())
    max_blocks = int(nblk.max().item())
    perm = torch.randperm(NB, generator=_gen(cfg.seed, 11, "cpu")).to(torch.int32)
    block_table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        n = int(nblk[b])
        block_table[b, :n] = perm[off:off + n]
        off += n
    out = {"seq_lens": lens.to(device), "block_table": block_table.to(device), "NB": NB,
           "max_blocks": max_blocks}
    out["q"] = (torch.randn(B, cfg.Hq, cfg.d, generator=_gen(cfg.seed, 1, device), device=device) * s).to(el)
    out["k_cache"] = (torch.randn(NB, bs, cfg.G, cfg.d, generator=_gen(cfg.seed, 2, device), device=device) * s).to(el)
    out["v_cache"] = (torch.randn(NB, bs, cfg.G, cfg.d, generator=_gen(cfg.seed, 3, device), device=device) * s).to(el)
    qi = torch.randn(B, cfg.HI, cfg.dI, generator=_gen(cfg.seed, 4, device), device=device)
    ki = torch.randn(NB * bs, cfg.dI, generator=_gen(cfg.seed, 5, device), device=device)
    out["w"] = torch.rand(B, cfg.HI, generator=_gen(cfg.seed, 7, device), device=device)
    out["q_idx"], out["q_scale"] = quantize_e4m3_per_token(qi)
    codes, scale = quantize_e4m3_per_token(ki)
    out["kidx_cache"] = codes.reshape(NB, bs, cfg.dI)
    out["kidx_scale"] = scale.reshape(NB, bs)
    return out


def packed_lengths(n: int, Lmin: int, Lmax: int, seed: int) -> list:
    """Seeded sequence lengths for a packed batch, uniform in [Lmin, Lmax]."""
    g = _gen(seed, 12, "cpu")
    return torch.randint(Lmin, Lmax + 1, (n,), generator=g).tolist()


def packed_prefill_inputs(cfg: PrefillConfig, lens, device="cpu") -> dict:
    """A packed batch: sequence i is ``prefill_inputs`` of ``cfg`` with L = lens[i] and seed
    cfg.seed + i, the sequences concatenated along the token dimension.  Adds ``cu_seqlens``
    (a list of len(lens) + 1 offsets)."""
    parts = [prefill_inputs(dataclasses.replace(cfg, L=int(n), seed=cfg.seed + i), device)
             for i, n in enumerate(lens) if n > 0]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    out = {"cu_seqlens": cu}
    for key in ("q", "k", "v", "q_idx", "q_scale", "w", "k_idx", "k_scale"):
        if parts and parts[0][key] is not None:
            out[key] = torch.cat([p[key] for p in parts]).contiguous()
        else:
            out[key] = None
    return out


def scaled(cfg, **changes):
    """A copy of ``cfg`` with some fields replaced (smaller test variants)."""
    return dataclasses.replace(cfg, **changes)


def relu_dominated_indexer_inputs(L: int, HI: int = 64, seed: int = 0, n_zero: int = 40,
                                  device="cpu") -> dict:
    """Indexer inputs whose dot products are mostly negative, so that ReLU zeroes most heads.

    A shared direction u ~ N(0, I) is added to every query head (q^I[t, j] = u + N(0, I)) and
    key s points against it by a seeded amount: k^I[s] = -lambda_s u / |u| + N(0, I) with
    lambda_s ~ U(0, 5).  For a typical pair from about half to all of its head dot products
    are negative, and about half of all pairs score exactly 0.  The first ``n_zero`` tokens
    have element-wise positive queries and element-wise negative keys, so among them every
    dot product is negative and every score is exactly 0; two of them have all-zero keys.
    w ~ U(0, 1).  FP8 codes as for the other workloads."""
    gen = lambda i: _gen(seed, 40 + i, device)
    u = torch.randn(128, generator=gen(0), device=device)
    qi = u + torch.randn(L, HI, 128, generator=gen(1), device=device)
    lam = torch.rand(L, 1, generator=gen(2), device=device) * 5.0
    ki = -lam * (u / u.norm()) + torch.randn(L, 128, generator=gen(3), device=device)
    z = min(n_zero, L)
    qi[:z] = torch.randn(z, HI, 128, generator=gen(4), device=device).abs()
    ki[:z] = -torch.randn(z, 128, generator=gen(5), device=device).abs()
    if z > 3:
        ki[1] = 0.0
        ki[z - 2] = 0.0
    out = {"w": torch.rand(L, HI, generator=gen(6), device=device)}
    out["q_idx"], out["q_scale"] = quantize_e4m3_per_token(qi)
    out["k_idx"], out["k_scale"] = quantize_e4m3_per_token(ki)
    return out
