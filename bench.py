#!/usr/bin/env python3
"""Benchmark of the DSA layer on one MI355X.

One step = one full causal prefill of a 128K-token sequence through the DSA
layer (FP8 lightning indexer -> top-k (k = 2048) -> GQA sparse attention),
processed in 8K-query chunks, on seeded synthetic inputs already resident in
HBM, through the one-call entry point dsa_prefill.  ``value`` is prefill
tokens per second of that call.  The paged decode step (64 sequences at
256K, and at lengths drawn from 32K..256K) is timed in a second region and
reported under ``decode``, with the step before it (the new token's indexer
query quantised to FP8 and its K/V/k^I appended into the paged caches) timed
alone and together with the decode step.

The same prefill is also run through the separate entry points (indexer over
full score rows, top-k, attention) with HIP events recorded on the launch
stream around every launch: ``kernels`` gives each kernel's average duration
and its algorithmic rate (FP8 FLOPs for the indexer, bytes for top-k and the
attention gather); the dominant kernel, the attention, which both paths run
identically, is reported as ``roofline``.  Both paths must give identical
index sets, and identical outputs outside the 16-row blocks of whole-prefix rows (which the
one-call path sends to the deduplicated attention; ``fused_vs_staged``).  The CPU oracle, timed on a stratified sample of
query rows, is reported as ``cpu_baseline``.  Packed batches through dsa_prefill_varlen (16
sequences of 2K..14K tokens, 64 of 1K..4K, 256 of 512) are reported under ``packed_prefill``,
and one sparse-adaptation
training step of the 32K layer (indexer scores at the selected positions, attention forward
with log-sum-exp, attention backward with the fused indexer loss, indexer backward) under
``train_step``.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"fp8": 5.0e15, "bf16": 2.5e15, "hbm": 8.0e12}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="prefill_128k_clustered")
    p.add_argument("--decode-workloads", default="decode_paged_64x256k,decode_paged_64x32k-256k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=960)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-packed", action="store_true")
    p.add_argument("--decode-only", action="store_true",
                   help="only the decode workloads (for counter collection on the decode kernels)")
    p.add_argument("--no-frames", action="store_true",
                   help="skip the frame-structured 128K prefill (dedup on and off)")
    p.add_argument("--no-prefill-256k", action="store_true",
                   help="skip the 256K multimodal prefill line")
    p.add_argument("--no-train", action="store_true")
    p.add_argument("--no-warmup-stage", action="store_true",
                   help="skip the dense warm-up training step")
    p.add_argument("--profile-kernel", choices=["index", "topk", "attn", "train", "warmup"], default=None,
                   help="profiling driver: run only this kernel on one chunk of the workload "
                        "(--profile-chunk, default the last) --profile-reps times, print nothing else; "
                        "'train': only the 32K training step, printing its JSON record")
    p.add_argument("--profile-chunk", type=int, default=-1)
    p.add_argument("--profile-reps", type=int, default=2)
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB first: the known-size "
                        "reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return p.parse_args()


def prefill_work(cfg):
    """Algorithmic work of each kernel for one chunked prefill (per chunk lists)."""
    L, k, C = cfg.L, cfg.k, cfg.chunk or cfg.L
    chunks = []
    for r0 in range(0, L, C):
        r1 = min(L, r0 + C)
        pairs = (r1 * (r1 + 1) - r0 * (r0 + 1)) // 2          # sum_{t=r0}^{r1-1} (t+1)
        n_sel = sum(min(k, t + 1) for t in range(r0, r1))
        long_rows = sum(1 for t in range(r0, r1) if t + 1 > k)
        pairs_long = sum(t + 1 for t in range(r0, r1) if t + 1 > k)
        chunks.append({
            "index_flop": 2 * cfg.HI * cfg.dI * pairs,
            # top-k reads each causal score of a row that needs selection once, writes k indices
            "topk_bytes": 4 * pairs_long + 4 * k * (r1 - r0),
            # gather of K and V rows of every selected position for all groups + q in + out
            "attn_bytes": n_sel * cfg.G * cfg.d * 2 * 2 + (r1 - r0) * cfg.Hq * cfg.d * 2 * 2,
            "attn_flop": 4 * n_sel * cfg.Hq * cfg.d,
            "rows": r1 - r0, "long_rows": long_rows,
        })
    return chunks


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when there is none for this workload or the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            entries = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if isinstance(entries, dict):
        entries = [entries]
    for entry in entries or []:
        if entry.get("workload") != workload:
            continue
        src = os.path.join(ROOT, "long_context_sparse_02_amd", "csrc", entry["source"])
        with open(src, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != entry["source_sha256"]:
                return None
        return entry["bytes_per_launch"]
    return None


def counter_roofline(kern, name, workload):
    """The roofline of kernel `name` (an entry of run_prefill_bench's per-kernel table): for an
    HBM-bound kernel with fresh committed counters, achieved = the counters' HBM bytes per launch
    / the launch's measured duration (what the memory interface carried); the algorithmic rate
    (the method's bytes or FLOPs per launch / duration) is kept beside it.  Without counters for
    this kernel source and workload, achieved is the algorithmic rate."""
    r = kern[name]
    traffic = measured_traffic(name, workload)
    algo = {"achieved": r["achieved"], "frac": r["frac"], "work_per_launch": r["work_per_launch"]}
    out = {"bound": r["bound"], "peak": r["peak"], "unit": r["unit"], "traffic": traffic,
           "kernel": name, "avg_launch_ms": r["avg_launch_ms"], "algorithmic": algo}
    if r["bound"] == "hbm" and traffic:
        achieved = traffic / (r["avg_launch_ms"] * 1e-3) / 1e9
        out.update(achieved=round(achieved, 2), frac=round(achieved / r["peak"], 4), basis="counters")
    else:
        out.update(achieved=r["achieved"], frac=r["frac"], basis="algorithmic")
    return out


def run_prefill_bench(args, dsa, W, torch, workload=None):
    cfg = W.ALL[workload or args.workload]
    dev = "cuda"
    log("generating", cfg.name)
    x = W.prefill_inputs(cfg, dev)
    torch.cuda.synchronize()
    L, k, C = cfg.L, cfg.k, cfg.chunk or cfg.L
    ld = (L + 3) // 4 * 4
    scores = torch.empty(C, ld, dtype=torch.float32, device=dev)
    idx = torch.empty(L, k, dtype=torch.int32, device=dev)
    out = torch.empty_like(x["q"])
    stream = torch.cuda.current_stream()
    s_ptr = stream.cuda_stream
    n_chunks = (L + C - 1) // C
    iws_n = dsa.dsa_index_scores_workspace_size(C, cfg.HI, cfg.dI, dsa.DSA_FP8_E4M3)
    iws = dsa.workspace(iws_n)

    def step(events=None):
        for c, r0 in enumerate(range(0, L, C)):
            rows = min(C, L - r0)
            tk = r0 + rows
            sl = slice(r0, r0 + rows)
            ev = events[c] if events else None
            if ev: ev[0].record(stream)
            dsa.dsa_index_scores(x["q_idx"][sl], x["q_scale"][sl], x["w"][sl], x["k_idx"], x["k_scale"],
                                 dsa.DSA_FP8_E4M3, rows, tk, cfg.HI, cfg.dI, r0, scores, ld, iws,
                                 iws_n, stream)
            if ev: ev[1].record(stream)
            dsa.dsa_topk(scores, ld, rows, tk, r0, k, idx[sl], None, 0, stream)
            if ev: ev[2].record(stream)
            dsa.dsa_sparse_gqa_attn(x["q"][sl], x["k"], x["v"], dsa.DSA_BF16, tk, None, 0, 0, None,
                                    None, idx[sl], rows, k, cfg.Hq, cfg.G, cfg.d, cfg.sm_scale,
                                    out[sl], None, 0, stream)
            if ev: ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_chunks)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    # per-kernel average durations (per launch) over the timed steps
    dur = {"index": [], "topk": [], "attn": []}
    for s in range(args.steps):
        for c in range(n_chunks):
            e = events[s][c]
            dur["index"].append(e[0].elapsed_time(e[1]) * 1e-3)
            dur["topk"].append(e[1].elapsed_time(e[2]) * 1e-3)
            dur["attn"].append(e[2].elapsed_time(e[3]) * 1e-3)
    work = prefill_work(cfg)
    kern = {}
    tot = lambda key: sum(w[key] for w in work)
    for name, key, unit, peak, bound in (("index", "index_flop", "TFLOP/s", PEAK["fp8"], "mfma"),
                                         ("topk", "topk_bytes", "GB/s", PEAK["hbm"], "hbm"),
                                         ("attn", "attn_bytes", "GB/s", PEAK["hbm"], "hbm")):
        per_launch_work = tot(key) / n_chunks
        avg = sum(dur[name]) / len(dur[name])
        scale = 1e12 if unit == "TFLOP/s" else 1e9
        achieved = per_launch_work / avg / scale
        kern[name] = {"bound": bound, "achieved": round(achieved, 2), "peak": peak / scale,
                      "unit": unit, "frac": round(achieved * scale / peak, 4),
                      "avg_launch_ms": round(avg * 1e3, 4), "launches": len(dur[name]),
                      "ms_per_step": round(sum(dur[name]) / args.steps * 1e3, 3),
                      "work_per_launch": per_launch_work}
    # the one-call entry point on the same inputs: the timed step
    del scores
    ws = dsa.workspace(dsa.dsa_prefill_workspace_size(L, 0, C, k))
    out2 = torch.empty_like(out)
    idx2 = torch.empty_like(idx)
    for _ in range(max(1, args.warmup)):
        dsa.dsa_prefill(x["q"], x["k"], x["v"], dsa.DSA_BF16, x["q_idx"], x["q_scale"], x["w"],
                        x["k_idx"], x["k_scale"], dsa.DSA_FP8_E4M3, L, 0, cfg.Hq, cfg.G, cfg.d,
                        cfg.HI, cfg.dI, k, cfg.sm_scale, C, out2, idx2, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        dsa.dsa_prefill(x["q"], x["k"], x["v"], dsa.DSA_BF16, x["q_idx"], x["q_scale"], x["w"],
                        x["k_idx"], x["k_scale"], dsa.DSA_FP8_E4M3, L, 0, cfg.Hq, cfg.G, cfg.d,
                        cfg.HI, cfg.dI, k, cfg.sm_scale, C, out2, idx2, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    fused_ms = (time.perf_counter() - t1) / args.steps * 1e3
    # rows in 16-row blocks of whole prefixes take the deduplicated attention in dsa_prefill (the
    # same terms, other rounding); everything else must be bitwise the staged path's
    lim = L if L <= k else (k // 16) * 16
    same = {"idx_equal": bool(torch.equal(idx, idx2)),
            "out_equal_beyond_prefix_blocks": bool(torch.equal(out[lim:], out2[lim:])),
            "prefix_block_rows": lim,
            "prefix_block_max_abs_diff": float((out[:lim].float() - out2[:lim].float()).abs().max())}
    del ws
    return cfg, x, idx, out, ms_step, kern, fused_ms, same


def run_prefill_256k_bench(args, dsa, W, torch):
    """The 256K multimodal prefill (16K-row chunks; its K/V, 512 MiB, exceed the 256 MiB
    last-level cache): fused tokens/s and each kernel's rate against its roofline."""
    steps = max(1, min(args.steps, 3))
    a2 = argparse.Namespace(**vars(args))
    a2.steps, a2.warmup = steps, 1
    cfg, x, idx, out, ms_step, kern, fused_ms, same = run_prefill_bench(a2, dsa, W, torch,
                                                                        "prefill_256k_multimodal")
    res = {"workload": cfg.name, "tokens": cfg.L, "chunk_rows": cfg.chunk, "steps": steps,
           "ms_per_step": round(fused_ms, 3), "tokens_per_s": round(cfg.L / (fused_ms * 1e-3), 1),
           "staged_ms_per_step": round(ms_step, 3),
           "kernels": {n: dict({kk: v[kk] for kk in ("avg_launch_ms", "ms_per_step", "achieved", "unit",
                                                     "frac")},
                               roofline=counter_roofline(kern, n, cfg.name)) for n, v in kern.items()},
           "fused_vs_staged": same}
    del x, idx, out
    torch.cuda.empty_cache()
    return res


def run_frames_bench(args, dsa, W, torch):
    """The 128K prefill with frame-structured indexer queries (adjacent queries of a frame select
    mostly the same keys, the regime where adjacent-query dedup pays): the fused prefill, then on
    the same selection the per-query attention of three chunks against the deduplicated one
    (every 16-row block on the union; and the switch, which takes the union only where it is
    small)."""
    cfg = W.scaled(W.PREFILL_128K, queries="frames", query_std=0.25)
    log("generating", cfg.name, "(frame-structured queries)")
    x = W.prefill_inputs(cfg, "cuda")
    L, C, k = cfg.L, cfg.chunk, cfg.k
    stream = torch.cuda.current_stream()
    out = torch.empty_like(x["q"])
    idx = torch.empty(L, k, dtype=torch.int32, device="cuda")
    ws = dsa.workspace(dsa.dsa_prefill_workspace_size(L, 0, C, k))
    run = lambda: dsa.dsa_prefill(x["q"], x["k"], x["v"], dsa.DSA_BF16, x["q_idx"], x["q_scale"], x["w"],
                                  x["k_idx"], x["k_scale"], dsa.DSA_FP8_E4M3, L, 0, cfg.Hq, cfg.G, cfg.d,
                                  cfg.HI, cfg.dI, k, cfg.sm_scale, C, out, idx, ws, ws.numel(), stream)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    fused_ms = timed(run, max(1, min(args.steps, 3)))
    del ws
    chunks = {}
    o2 = torch.empty(C, cfg.Hq, cfg.d, dtype=torch.bfloat16, device="cuda")
    for c in (0, 8, 15):
        r0 = c * C
        sl = slice(r0, r0 + C)
        qc, ic = x["q"][sl], idx[sl]
        pq = lambda: dsa.dsa_sparse_gqa_attn(qc, x["k"], x["v"], dsa.DSA_BF16, r0 + C, None, 0, 0, None,
                                             None, ic, C, k, cfg.Hq, cfg.G, cfg.d, cfg.sm_scale, o2,
                                             None, 0, stream)
        nws = dsa.dsa_sparse_gqa_attn_dedup_workspace_size(C, r0, k)
        dws = dsa.workspace(nws)
        dd = lambda mode: dsa.dsa_sparse_gqa_attn_dedup(qc, x["k"], x["v"], r0 + C, ic, C, r0, k, cfg.Hq,
                                                        cfg.G, cfg.d, cfg.sm_scale, mode, o2, dws, nws,
                                                        stream)
        chunks["chunk_%d" % c] = {"per_query_ms": round(timed(pq, 3), 3),
                                  "dedup_every_block_ms": round(timed(lambda: dd(1), 3), 3),
                                  "dedup_switch_ms": round(timed(lambda: dd(0), 3), 3),
                                  "adjacent16_union": round(adjacent_union(idx[r0:r0 + C], C, min(k, C // 2)
                                                                           if c == 0 else k,
                                                                           seed=c), 1)
                                  if c else None}
        del dws
    res = {"workload": cfg.name + "_frames", "queries": "frames", "query_std": cfg.query_std,
           "ms_per_step": round(fused_ms, 3), "tokens_per_s": round(L / (fused_ms * 1e-3), 1),
           "adjacent16_union": round(adjacent_union(idx, L, k), 1), "attention_by_chunk": chunks}
    del x, idx, out, o2
    torch.cuda.empty_cache()
    return res


def adjacent_union(idx, L, k, groups=64, width=16, seed=0):
    """Mean number of distinct positions selected by `width` adjacent queries, over
    `groups` seeded groups of rows with t >= k (the structure statistic of adjacent-query
    Top-KV deduplication)."""
    import torch
    g = torch.Generator().manual_seed(seed)
    starts = torch.randint(k, L - width, (groups,), generator=g).tolist()
    sizes = []
    for s0 in starts:
        sel = idx[s0:s0 + width].reshape(-1)
        sizes.append(int(torch.unique(sel[sel >= 0]).numel()))
    return sum(sizes) / len(sizes)


def run_profile_kernel(args, dsa, W, torch):
    """One kernel of the staged prefill, on one chunk, for counter collection."""
    cfg = W.ALL[args.workload]
    x = W.prefill_inputs(cfg, "cuda")
    L, k, C = cfg.L, cfg.k, cfg.chunk or cfg.L
    n_chunks = (L + C - 1) // C
    c = args.profile_chunk % n_chunks
    r0 = c * C
    rows = min(C, L - r0)
    tk = r0 + rows
    sl = slice(r0, r0 + rows)
    ld = (L + 3) // 4 * 4
    scores = torch.empty(rows, ld, dtype=torch.float32, device="cuda")
    idx = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    out = torch.empty_like(x["q"][sl])
    iws_n = dsa.dsa_index_scores_workspace_size(rows, cfg.HI, cfg.dI, dsa.DSA_FP8_E4M3)
    iws = dsa.workspace(iws_n)
    stream = torch.cuda.current_stream()
    index = lambda: dsa.dsa_index_scores(x["q_idx"][sl], x["q_scale"][sl], x["w"][sl], x["k_idx"],
                                         x["k_scale"], dsa.DSA_FP8_E4M3, rows, tk, cfg.HI, cfg.dI, r0,
                                         scores, ld, iws, iws_n, stream)
    topk = lambda: dsa.dsa_topk(scores, ld, rows, tk, r0, k, idx, None, 0, stream)
    attn = lambda: dsa.dsa_sparse_gqa_attn(x["q"][sl], x["k"], x["v"], dsa.DSA_BF16, tk, None, 0, 0,
                                           None, None, idx, rows, k, cfg.Hq, cfg.G, cfg.d,
                                           cfg.sm_scale, out, None, 0, stream)
    if args.profile_kernel in ("topk", "attn"):
        index()
    if args.profile_kernel == "attn":
        topk()
    run = {"index": index, "topk": topk, "attn": attn}[args.profile_kernel]
    for _ in range(args.profile_reps):
        run()
    torch.cuda.synchronize()
    log("profiled %s on chunk %d (rows %d..%d) x %d" % (args.profile_kernel, c, r0, r0 + rows - 1,
                                                      args.profile_reps))


def run_decode_bench(args, dsa, W, torch, name):
    cfg = W.ALL[name]
    log("generating", cfg.name)
    x = W.decode_inputs(cfg, "cuda")
    out = torch.empty_like(x["q"])
    n = dsa.dsa_decode_workspace_size(cfg.B, x["max_blocks"], cfg.block, cfg.k, cfg.Hq, cfg.d)
    ws = dsa.workspace(n)
    stream = torch.cuda.current_stream()

    def step():
        dsa.dsa_decode(x["q"], x["q_idx"], x["q_scale"], x["w"], x["kidx_cache"], x["kidx_scale"],
                       x["k_cache"], x["v_cache"], dsa.DSA_BF16, x["block_table"], x["seq_lens"],
                       cfg.B, x["NB"], x["max_blocks"], cfg.block, cfg.Hq, cfg.G, cfg.d, cfg.HI,
                       cfg.dI, cfg.k, cfg.sm_scale, out, None, ws, ws.numel(), stream)
    for _ in range(max(2, args.warmup)):
        step()
    torch.cuda.synchronize()
    steps = max(10, args.steps * 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    us_step = e0.elapsed_time(e1) / steps * 1e3

    # the step before decode: the new token's indexer query quantised (one scale per token
    # over its H^I x d_I values) and its K/V/k^I appended at position len - 1
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed + 1000)
    qi_f = torch.randn(cfg.B, cfg.HI * cfg.dI, generator=gen, device="cuda").bfloat16()
    kidx_f = torch.randn(cfg.B, cfg.dI, generator=gen, device="cuda").bfloat16()
    k_new = torch.randn(cfg.B, cfg.G, cfg.d, generator=gen, device="cuda").bfloat16()
    v_new = torch.randn(cfg.B, cfg.G, cfg.d, generator=gen, device="cuda").bfloat16()
    pos = (x["seq_lens"] - 1).contiguous()
    q_idx_flat = x["q_idx"].view(cfg.B, -1)

    def prep():
        dsa.dsa_quantize_e4m3(qi_f, dsa.DSA_BF16, cfg.B, cfg.HI * cfg.dI, q_idx_flat, x["q_scale"],
                              stream)
        dsa.dsa_cache_append(k_new, v_new, dsa.DSA_BF16, kidx_f, dsa.DSA_BF16, pos,
                             x["block_table"], cfg.B, x["NB"], x["max_blocks"], cfg.block, cfg.G,
                             cfg.d, cfg.dI, x["k_cache"], x["v_cache"], x["kidx_cache"],
                             x["kidx_scale"], stream)
    timed = {}
    for what, fn in (("prep", prep), ("serving", lambda: (prep(), step()))):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        timed[what] = e0.elapsed_time(e1) / steps * 1e3
    lens = x["seq_lens"].long().cpu()
    # algorithmic bytes: indexer keys (codes + scale) + score write/read + gather + q/out
    key_bytes = int(lens.sum()) * (cfg.dI + 4)
    score_bytes = int(lens.sum()) * 8
    gather = int(torch.clamp(lens, max=cfg.k).sum()) * cfg.G * cfg.d * 2 * 2
    qo = cfg.B * (cfg.Hq * cfg.d * 2 * 2 + cfg.HI * cfg.dI + cfg.HI * 4)
    total = key_bytes + score_bytes + gather + qo
    res = {"workload": cfg.name, "us_per_step": round(us_step, 2),
           "us_per_token": round(us_step / cfg.B, 3),
           "mean_len": float(lens.float().mean()), "algorithmic_bytes": total,
           "achieved_GBps": round(total / (us_step * 1e-6) / 1e9, 1),
           "hbm_frac": round(total / (us_step * 1e-6) / PEAK["hbm"], 4),
           "us_quantize_and_append": round(timed["prep"], 2),
           "us_per_serving_step": round(timed["serving"], 2)}
    del x, ws
    torch.cuda.empty_cache()
    return res


PACKED = [  # (name, sequences, shortest, longest, seed)
    ("prefill_packed_16x2k-14k", 16, 2048, 14336, 1010),
    ("prefill_packed_64x1k-4k", 64, 1024, 4096, 1011),
    ("prefill_packed_256x512", 256, 512, 512, 1012),
]


def run_packed_bench(args, dsa, W, torch, name, n_seq, lmin, lmax, seed):
    """Packed variable-length prefill: n_seq sequences of lmin..lmax tokens (seeded, clustered
    keys, the 128K layer's shapes), one dsa_prefill_varlen call per step."""
    cfg = W.scaled(W.PREFILL_128K, L=1, seed=seed)
    lens = W.packed_lengths(n_seq, lmin, lmax, cfg.seed)
    log("generating packed batch", name)
    x = W.packed_prefill_inputs(cfg, lens, "cuda")
    cu = x["cu_seqlens"]
    T = cu[-1]
    max_len = max(lens)
    out = torch.empty_like(x["q"])
    n = dsa.dsa_prefill_workspace_size(max_len, 0, cfg.chunk, cfg.k)
    ws = dsa.workspace(n)
    stream = torch.cuda.current_stream()

    def step():
        dsa.dsa_prefill_varlen(x["q"], x["k"], x["v"], dsa.DSA_BF16, x["q_idx"], x["q_scale"],
                               x["w"], x["k_idx"], x["k_scale"], dsa.DSA_FP8_E4M3, cu, len(lens),
                               cfg.Hq, cfg.G, cfg.d, cfg.HI, cfg.dI, cfg.k, cfg.sm_scale,
                               cfg.chunk, out, None, ws, ws.numel(), stream)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    steps = max(3, args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    res = {"workload": name, "sequences": len(lens), "tokens": T,
           "max_len": max_len, "ms_per_step": round(ms, 3),
           "tokens_per_s": round(T / (ms * 1e-3), 1)}
    del x, ws, out
    torch.cuda.empty_cache()
    return res


def run_train_bench(args, dsa, W, torch):
    """One sparse-adaptation training step of the layer at 32K (report section 2.3.3): the
    indexer scores at the selected positions, the attention forward with its log-sum-exp,
    the attention backward with the fused indexer loss, and the indexer backward."""
    cfg = W.PREFILL_32K
    log("generating", cfg.name, "(training step)")
    x = W.prefill_inputs(cfg, "cuda")
    L, k, G = cfg.L, cfg.k, cfg.G
    _, idx = dsa.prefill(x["q"], x["k"], x["v"], x["q_idx"], x["q_scale"], x["w"], x["k_idx"],
                         x["k_scale"], k, cfg.sm_scale, return_idx=True)
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed + 2000)
    dout = torch.randn(x["q"].shape, generator=gen, device="cuda").bfloat16()
    out = torch.empty_like(x["q"])
    lse = torch.empty(L, cfg.Hq, dtype=torch.float32, device="cuda")
    vals = torch.empty(L, k, dtype=torch.float32, device="cuda")
    dq = torch.empty_like(x["q"])
    dk = torch.empty(x["k"].shape, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    kl = torch.empty(L, dtype=torch.float32, device="cuda")
    dI = torch.empty(L, k, dtype=torch.float32, device="cuda")
    dqi = torch.empty(x["q_idx"].shape, dtype=torch.float32, device="cuda")
    dw = torch.empty(x["w"].shape, dtype=torch.float32, device="cuda")
    dki = torch.empty(x["k_idx"].shape, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    bws = dsa.workspace(dsa.dsa_sparse_gqa_attn_bwd_workspace_size(L, k, G, L))
    iws = dsa.workspace(dsa.dsa_index_scores_at_bwd_workspace_size(L, L, cfg.HI, k))
    BF, F8 = dsa.DSA_BF16, dsa.DSA_FP8_E4M3
    parts = {
        "index_at": lambda: dsa.dsa_index_scores_at(
            x["q_idx"], x["q_scale"], x["w"], x["k_idx"], x["k_scale"], F8, L, L, cfg.HI, cfg.dI,
            idx, k, vals, stream),
        "attn_fwd_lse": lambda: dsa.dsa_sparse_gqa_attn_lse(
            x["q"], x["k"], x["v"], BF, L, idx, L, k, cfg.Hq, G, cfg.d, cfg.sm_scale, out, lse,
            None, 0, stream),
        "attn_bwd_kl": lambda: (dk.zero_(), dv.zero_(), dsa.dsa_sparse_gqa_attn_bwd(
            x["q"], x["k"], x["v"], BF, L, idx, L, k, cfg.Hq, G, cfg.d, cfg.sm_scale, out, dout,
            lse, dq, dk, dv, vals, kl, dI, bws, bws.numel(), stream=stream)),
        "index_at_bwd": lambda: (dki.zero_(), dsa.dsa_index_scores_at_bwd(
            x["q_idx"], x["q_scale"], x["w"], x["k_idx"], x["k_scale"], F8, L, L, cfg.HI, cfg.dI,
            idx, k, dI, dqi, dw, dki, iws, iws.numel(), stream=stream)),
    }
    for _ in range(max(1, args.warmup)):
        for f in parts.values():
            f()
    torch.cuda.synchronize()
    reps = max(2, args.steps)
    ms = {}
    for name, f in parts.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / reps
    n_sel = int(torch.clamp(torch.arange(1, L + 1, device="cuda"), max=k).sum())
    # attention backward, staged: per selected pair and KV group the K and V rows gathered
    # (2 x 256 B) and the dK / dV contribution written and read back (2 x 1 KiB); indexer
    # backward, staged: per selected pair the key row (128 B + scale) gathered and the dk^I
    # contribution written and read back (2 x 512 B)
    attn_bytes = n_sel * G * (2 * cfg.d * 2 + 2 * 2 * cfg.d * 4)
    ix_bytes = n_sel * (cfg.dI + 4 + 2 * cfg.dI * 4)
    step = sum(ms.values())
    res = {"workload": cfg.name + "_train_step", "tokens": L, "selected_pairs": n_sel,
           "ms": {n: round(v, 3) for n, v in ms.items()}, "ms_per_step": round(step, 3),
           "tokens_per_s": round(L / (step * 1e-3), 1),
           "attn_bwd_bytes": attn_bytes,
           "attn_bwd_hbm_frac": round(attn_bytes / (ms["attn_bwd_kl"] * 1e-3) / PEAK["hbm"], 4),
           "index_bwd_bytes": ix_bytes,
           "index_bwd_hbm_frac": round(ix_bytes / (ms["index_at_bwd"] * 1e-3) / PEAK["hbm"], 4),
           "mean_kl": round(float(kl.mean()), 5)}
    del x, idx, out, lse, vals, dq, dk, dv, kl, dI, dqi, dw, dki, dout, bws, iws
    torch.cuda.empty_cache()
    return res


def _dense_lse(q, k, G, sm_scale, torch, rows=256):
    """Natural-log softmax normaliser of every query head over its causal prefix, [L, Hq]
    float32 (fp32 products of the bf16 inputs, in blocks of query rows)."""
    L, Hq, d = q.shape
    hpg = Hq // G
    kf = k.float()                                        # [L, G, d]
    out = torch.empty(L, Hq, dtype=torch.float32, device=q.device)
    pos = torch.arange(L, device=q.device)
    for r0 in range(0, L, rows):
        r1 = min(L, r0 + rows)
        qf = q[r0:r1].float().view(r1 - r0, G, hpg, d).permute(1, 0, 2, 3).reshape(G, (r1 - r0) * hpg, d)
        kk = kf[:r1].permute(1, 2, 0).contiguous()        # [G, d, r1]
        s = torch.bmm(qf.contiguous(), kk).view(G, r1 - r0, hpg, r1) * sm_scale
        mask = pos[None, :r1] > pos[r0:r1, None]          # keys past each row's position
        s.masked_fill_(mask[None, :, None, :], float("-inf"))
        out[r0:r1] = torch.logsumexp(s, dim=-1).permute(1, 0, 2).reshape(r1 - r0, Hq)
    return out


def run_warmup_bench(args, dsa, W, torch):
    """One dense warm-up training step of the layer at 32K (report section 2.3.3): the indexer's
    full causal score rows, the warm-up loss with dL/dI written over them (the heads'
    log-sum-exp computed, not given), and the dense indexer backward."""
    cfg = W.PREFILL_32K
    log("generating", cfg.name, "(warm-up step)")
    x = W.prefill_inputs(cfg, "cuda")
    L, G, HI, dI, Hq, d = cfg.L, cfg.G, cfg.HI, cfg.dI, cfg.Hq, cfg.d
    ld = (L + 3) // 4 * 4
    scores = torch.empty(L, ld, dtype=torch.float32, device="cuda")
    kl = torch.empty(L, dtype=torch.float32, device="cuda")
    dqi = torch.empty(x["q_idx"].shape, dtype=torch.float32, device="cuda")
    dw = torch.empty(x["w"].shape, dtype=torch.float32, device="cuda")
    dki = torch.empty(x["k_idx"].shape, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    F8 = dsa.DSA_FP8_E4M3
    n_ix = dsa.dsa_index_scores_workspace_size(L, HI, dI, F8)
    ixws = dsa.workspace(n_ix) if n_ix else None
    bws = dsa.workspace(dsa.dsa_index_scores_bwd_dense_workspace_size(L, L, HI))
    parts = {
        "index_scores": lambda: dsa.dsa_index_scores(
            x["q_idx"], x["q_scale"], x["w"], x["k_idx"], x["k_scale"], F8, L, L, HI, dI, 0,
            scores, ld, ixws, n_ix, stream),
        "warmup_kl": lambda: dsa.dsa_indexer_warmup_kl(
            x["q"], x["k"], dsa.DSA_BF16, L, L, 0, Hq, G, d, cfg.sm_scale, None, scores, ld, kl,
            stream),
        "index_bwd_dense": lambda: (dki.zero_(), dsa.dsa_index_scores_bwd_dense(
            x["q_idx"], x["q_scale"], x["w"], x["k_idx"], x["k_scale"], F8, L, L, HI, dI, 0,
            scores, ld, dqi, dw, dki, bws, bws.numel(), stream)),
    }
    # the parts run in order on the stream (the loss consumes the scores, the backward dI), so
    # each is timed inside full steps: events around every part of every step
    for _ in range(max(1, args.warmup)):
        for f in parts.values():
            f()
    torch.cuda.synchronize()
    reps = max(2, args.steps)
    ev = {n: [] for n in parts}
    for _ in range(reps):
        for name, f in parts.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            f()
            e1.record(stream)
            ev[name].append((e0, e1))
    torch.cuda.synchronize()
    ms = {n: sum(a.elapsed_time(b) for a, b in v) / reps for n, v in ev.items()}
    # the loss again with the heads' log-sum-exp supplied (as a dense attention forward
    # returns it; computed here once, untimed, in fp32): one q.K pass instead of two
    lse = _dense_lse(x["q"], x["k"], G, cfg.sm_scale, torch)
    given = lambda: dsa.dsa_indexer_warmup_kl(
        x["q"], x["k"], dsa.DSA_BF16, L, L, 0, Hq, G, d, cfg.sm_scale, lse, scores, ld, kl, stream)
    ev_g = []
    for _ in range(reps):
        parts["index_scores"]()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        given()
        e1.record(stream)
        ev_g.append((e0, e1))
    torch.cuda.synchronize()
    ms_given = sum(a.elapsed_time(b) for a, b in ev_g) / reps
    pairs = L * (L + 1) // 2
    # algorithmic work per causal pair: the indexer 2 H^I d_I FP8 FLOP; the loss the scores of
    # every query head, 2 Hq d bf16 FLOP (computed twice here: once for the log-sum-exp); the
    # backward x once more (FP8) and the two products with G (2 x 2 H^I d_I bf16 FLOP)
    ix_flop = pairs * 2 * HI * dI
    kl_flop = pairs * 2 * Hq * d
    bwd_f8, bwd_bf = pairs * 2 * HI * dI, pairs * 4 * HI * dI
    step = sum(ms.values())
    res = {"workload": cfg.name + "_warmup_step", "tokens": L, "causal_pairs": pairs,
           "ms": {n: round(v, 3) for n, v in ms.items()}, "ms_per_step": round(step, 3),
           "tokens_per_s": round(L / (step * 1e-3), 1),
           "index_mfma_frac": round(ix_flop / (ms["index_scores"] * 1e-3) / PEAK["fp8"], 4),
           "kl_mfma_frac": round(kl_flop / (ms["warmup_kl"] * 1e-3) / PEAK["bf16"], 4),
           "warmup_kl_lse_given_ms": round(ms_given, 3),
           "kl_lse_given_mfma_frac": round(kl_flop / (ms_given * 1e-3) / PEAK["bf16"], 4),
           "bwd_mfma_frac": round((bwd_f8 / PEAK["fp8"] + bwd_bf / PEAK["bf16"])
                                  / (ms["index_bwd_dense"] * 1e-3), 4),
           "mean_kl": round(float(kl.mean()), 5)}
    del x, scores, kl, dqi, dw, dki, ixws, bws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args, cfg, x, torch):
    """The oracle on a stratified sample of query rows of the same workload."""
    import numpy as np
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import to_np
    L = cfg.L
    n = args.cpu_rows
    rows = np.array([int((i + 0.5) * L / n) for i in range(n)], np.int32)
    rt = torch.from_numpy(rows).long().to(x["q"].device)
    qi, qs, w = to_np(x["q_idx"][rt]), to_np(x["q_scale"][rt]), to_np(x["w"][rt])
    ki, ks = to_np(x["k_idx"]), to_np(x["k_scale"])
    q, kk, vv = to_np(x["q"][rt]), to_np(x["k"]), to_np(x["v"])
    threads = oracle.num_threads()
    idx = np.empty((n, cfg.k), np.int32)
    from concurrent.futures import ThreadPoolExecutor

    def one(j):
        # one call per row keeps each row at its own causal length; rows run in parallel
        r = int(rows[j])
        s = oracle.index_scores(qi[j:j + 1], qs[j:j + 1], w[j:j + 1], ki[:r + 1], ks[:r + 1],
                                oracle.FP8_E4M3, q_pos0=r)
        sel, _ = oracle.topk(s, [r], cfg.k)
        return sel[0]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for j, sel in enumerate(ex.map(one, range(n))):
            idx[j] = sel
    oracle.sparse_gqa_attn(q, kk, vv, oracle.BF16, idx, cfg.Hq, cfg.G, cfg.sm_scale)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d query rows at positions (i+0.5)*L/%d of the %s workload (full indexer "
                      "over each row's prefix, top-k, attention), %.1f s wall" % (n, n, cfg.name, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the DSA layer here is a single-GPU build "
              "(no collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import long_context_sparse_02_amd as dsa
    import workloads as W
    dsa.load_library()
    if args.profile_kernel == "warmup":
        print(json.dumps(run_warmup_bench(args, dsa, W, torch)), flush=True)
        return
    if args.profile_kernel == "train":
        # the 32K training step alone (warm-up and timed repetitions as --warmup / --steps)
        print(json.dumps(run_train_bench(args, dsa, W, torch)), flush=True)
        return
    if args.profile_kernel:
        run_profile_kernel(args, dsa, W, torch)
        return
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.decode_only:
        print(json.dumps([run_decode_bench(args, dsa, W, torch, n)
                          for n in args.decode_workloads.split(",") if n]), flush=True)
        return
    cfg, x, idx, out, ms_step, kern, fused_ms, same = run_prefill_bench(args, dsa, W, torch)
    dom = max(kern, key=lambda n: kern[n]["ms_per_step"])
    roofline = counter_roofline(kern, dom, cfg.name)
    for name in kern:
        kern[name]["roofline"] = counter_roofline(kern, name, cfg.name)
    result = {
        "metric": "DSA layer tokens/s at 128K prefill + decode us/token at 256K, % of MI355X roofline",
        "value": round(cfg.L / (fused_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(fused_ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8+bf16",
        "data": "synthetic (seeded; clustered FP8 indexer keys, bf16 q/k/v)",
        "config": {"workload": cfg.name, "seq_len": cfg.L, "chunk_rows": cfg.chunk, "topk": cfg.k,
                   "Hq": cfg.Hq, "G": cfg.G, "d": cfg.d, "HI": cfg.HI, "dI": cfg.dI,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": kern,
        "staged_ms_per_step": round(ms_step, 3), "fused_vs_staged": same,
        "adjacent16_union": round(adjacent_union(idx, cfg.L, cfg.k), 1),
    }
    del x, idx, out
    torch.cuda.empty_cache()
    if not args.no_frames:
        result["frames_prefill"] = run_frames_bench(args, dsa, W, torch)
    if not args.no_prefill_256k:
        result["prefill_256k"] = run_prefill_256k_bench(args, dsa, W, torch)
    if not args.no_packed:
        result["packed_prefill"] = [run_packed_bench(args, dsa, W, torch, *p) for p in PACKED]
    if not args.no_train:
        result["train_step"] = run_train_bench(args, dsa, W, torch)
    if not args.no_warmup_stage:
        result["warmup_step"] = run_warmup_bench(args, dsa, W, torch)
    if not args.no_decode:
        result["decode"] = [run_decode_bench(args, dsa, W, torch, n)
                            for n in args.decode_workloads.split(",") if n]
    if not args.no_cpu_baseline:
        x = W.prefill_inputs(cfg, "cuda")
        result["cpu_baseline"] = cpu_baseline(args, cfg, x, torch)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
