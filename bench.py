"""Benchmark of the block-summary sparse decode step on one MI355X.

A step is one pass of the per-token hot path over the workload's batch:
select_blocks (block scores + top-k) then sparse_decode_attn (split-K
attention over the kept blocks + exact merge).  Block summaries are built once
when the cache is ingested and timed separately.

Timing: W untimed warmup steps, then exactly K timed steps between a
synchronize on both sides.  Before every step an untimed flush reads and
writes 1 GiB so that neither L2 nor the 256 MB Infinity Cache still holds the
previous step's KV: each step streams its kept KV from HBM.  Every call is
bracketed by HIP events recorded on the stream the kernels are launched on.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-decode attn queries·heads/s + achieved HBM GB/s at 128K ctx, 15% keep"
HBM_PEAK_GBS = 8000.0


def kv_bytes_per_token(n_layers, width, elem_bytes):
    """K and V bytes of one token: layers x (heads * head_dim) x bytes x 2."""
    return n_layers * width * elem_bytes * 2


def decode_bytes(cfg, n_keep):
    """Algorithmic bytes of the two calls of one decode step.

    select: the fp32 summaries of every block + q; attend: the kept K and V (bf16), q, the
    fp32 output and lse, and the index list.  Unselected KV and implementation scratch
    (scores, split partials) are not counted."""
    B, Hq, Hkv, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    nb = -(-cfg.seq_len // cfg.block_size)
    kept_tokens = min(n_keep * cfg.block_size, cfg.seq_len)
    q_bytes = B * Hq * d * 2
    sel = B * Hkv * nb * d * 4 + q_bytes
    att = (B * Hkv * kept_tokens * kv_bytes_per_token(1, d, 2) + q_bytes + B * Hq * d * 4
           + B * Hq * 4 + B * Hkv * n_keep * 4)
    return sel, att


def step_bytes(cfg, n_keep):
    """Algorithmic bytes of one step: both calls' bytes with q counted once."""
    sel, att = decode_bytes(cfg, n_keep)
    return sel + att - cfg.batch * cfg.n_q_heads * cfg.head_dim * 2


def partials_bytes(cfg, n_keep):
    """Algorithmic bytes of step S4 alone (the split-K partials kernel): 64 * d * 2 * 2 bytes of
    K and V per (batch, kv head, kept block), plus q and the index list.  The fp32 output is
    S5's; the partials are scratch."""
    B, Hq, Hkv, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    kept_tokens = min(n_keep * cfg.block_size, cfg.seq_len)
    return B * Hkv * kept_tokens * kv_bytes_per_token(1, d, 2) + B * Hq * d * 2 + B * Hkv * n_keep * 4


def measured_traffic(workload, field="traffic_bytes_per_launch"):
    """HBM bytes per launch from the committed counter summary (`field`: the whole
    sparse_decode_attn call, or the S4 kernel alone), or None when the summary is for another
    workload or the decode kernel's sources (kernels_decode.hip, then the device helpers
    bsa_device.h, hashed as one byte string) changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"decode_{workload}_hbm_traffic.md")
    csrc = os.path.join(ROOT, "long_context_block_summary_amd", "csrc")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and not line.startswith(("|", "#", "`")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    src = b"".join(open(os.path.join(csrc, f), "rb").read()
                   for f in ("kernels_decode.hip", "bsa_device.h"))
    sha = hashlib.sha256(src).hexdigest()[:16]
    if fields.get("kernel_source_sha256_prefix") != sha:
        return None
    return float(fields[field]) if field in fields else None


MFMA_BF16_PEAK_TFLOPS = 2500.0


def run_gpu(cfg, steps, warmup, flush_bytes=1 << 30, inputs=None):
    import numpy as np
    import torch

    import long_context_block_summary_amd as bsa
    from long_context_block_summary_amd import synth

    dev = torch.device("cuda:0")
    t = inputs if inputs is not None else synth.gen_decode(cfg)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to(t["q"]), to(t["k"]), to(t["v"])
    N, bs = cfg.seq_len, cfg.block_size
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    flush.zero_()

    # ingest: summaries (S1), cold
    summ = torch.empty((cfg.batch, cfg.n_kv_heads, -(-N // bs), cfg.head_dim),
                       dtype=torch.float32, device=dev)
    sum_ms = []
    for _ in range(3):
        flush.add_(1.0)
        e0, e1 = ev(), ev()
        e0.record(stream)
        bsa.build_block_summaries(k, N, bs, out_f32=summ)
        e1.record(stream)
        torch.cuda.synchronize()
        sum_ms.append(e0.elapsed_time(e1))

    cfgc = bsa.select_cfg(bs, cfg.n_sink, cfg.n_local, cfg.top_k, cfg.keep_ratio)
    n_keep = bsa.num_kept(-(-N // bs), cfgc)
    idx = torch.empty((cfg.batch, cfg.n_kv_heads, n_keep), dtype=torch.int32, device=dev)
    out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.batch, cfg.n_q_heads), dtype=torch.float32, device=dev)
    ws_sel = torch.empty(cfg.batch * cfg.n_kv_heads * (-(-N // bs)) * 4, dtype=torch.uint8,
                         device=dev)
    ws_dec = torch.zeros(max(16, bsa.decode_workspace_size(cfg.batch, cfg.n_q_heads,
                                                           cfg.n_kv_heads, cfg.head_dim, N,
                                                           n_keep)),
                         dtype=torch.uint8, device=dev)

    ws_step = torch.empty(bsa.decode_step_workspace_size(cfg.batch, cfg.n_q_heads,
                                                          cfg.n_kv_heads, cfg.head_dim, N, bs,
                                                          cfg.n_sink, cfg.n_local, cfg.top_k,
                                                          cfg.keep_ratio),
                          dtype=torch.uint8, device=dev)

    def one_call(e0=None, e2=None):
        """the step as one sparse_decode_step call (S2-S5; S3 and S5 inside the attention
        launch where the candidate count allows)"""
        st = torch.cuda.current_stream(dev)
        if e0 is not None:
            e0.record(st)
        bsa.sparse_decode_step(q, k, v, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k,
                               cfg.keep_ratio, block_idx=idx, out=out, lse=lse,
                               workspace=ws_step)
        if e2 is not None:
            e2.record(st)

    def step(e0=None, e1=None, e2=None, e3=None):
        """the step as its two calls, select_blocks then sparse_decode_attn (or the latter's
        two steps S4 and S5 as calls of their own)"""
        st = torch.cuda.current_stream(dev)
        if e0 is not None:
            e0.record(st)
        bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k, cfg.keep_ratio,
                          block_idx=idx, workspace=ws_sel)
        if e1 is not None:
            e1.record(st)
        if e3 is None:
            bsa.sparse_decode_attn(q, k, v, idx, N, bs, out=out, lse=lse, workspace=ws_dec)
            if e2 is not None:
                e2.record(st)
        else:  # the attention as its two steps, S4 (partials) and S5 (merge), timed apart
            bsa.sparse_decode_partials(q, k, v, idx, N, bs, workspace=ws_dec)
            e2.record(st)
            bsa.sparse_decode_merge(ws_dec, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads,
                                    cfg.head_dim, N, n_keep, bs, out=out, lse=lse)
            e3.record(st)

    for _ in range(warmup):
        flush.add_(1.0)
        step()
        flush.add_(1.0)
        one_call()
    # headline: the one-call step, events at the step boundaries only
    events = [(ev(), ev()) for _ in range(steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for e0, e2 in events:
        flush.add_(1.0)
        one_call(e0=e0, e2=e2)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    step_ms = [a.elapsed_time(b) for a, b in events]
    # the same step as the two calls (a timing event between them would cost the GPU a
    # few microseconds of idle time, so again only at the step boundaries)
    tevents = [(ev(), ev()) for _ in range(steps)]
    for e0, e2 in tevents:
        flush.add_(1.0)
        step(e0=e0, e2=e2)
    torch.cuda.synchronize()
    two_ms = [a.elapsed_time(b) for a, b in tevents]

    # per-call breakdown (separate passes with events between the calls): select + the
    # attention call; select + its two steps S4 and S5 as separate calls
    bevents = [(ev(), ev(), ev()) for _ in range(steps)]
    for e in bevents:
        flush.add_(1.0)
        step(*e)
    torch.cuda.synchronize()
    sel_ms = [a.elapsed_time(b) for a, b, _ in bevents]
    att_ms = [b.elapsed_time(c) for _, b, c in bevents]
    sevents = [(ev(), ev(), ev(), ev()) for _ in range(steps)]
    for e in sevents:
        flush.add_(1.0)
        step(*e)
    torch.cuda.synchronize()
    s4_ms = [b.elapsed_time(c) for _, b, c, _ in sevents]
    s5_ms = [c.elapsed_time(d) for _, _, c, d in sevents]

    # the same step captured once in a HIP graph and replayed (flush outside the graph)
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            one_call()  # warm the side stream once outside capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            one_call()
        torch.cuda.synchronize()
        gevents = [(ev(), ev()) for _ in range(steps)]
        for e0, e1 in gevents:
            flush.add_(1.0)
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = [a.elapsed_time(b) for a, b in gevents]
        del g
    except Exception as exc:  # report, never fall back silently
        graph_ms = f"capture failed: {exc!r}"

    # warm-cache (no flush) for reference only
    torch.cuda.synchronize()
    we = [(ev(), ev()) for _ in range(steps)]
    for e0, e2 in we:
        one_call(e0=e0, e2=e2)
    torch.cuda.synchronize()
    warm_ms = [a.elapsed_time(b) for a, b in we]
    return {
        "n_keep": n_keep,
        "sum_ms": sorted(sum_ms)[len(sum_ms) // 2],
        "sel_ms": sum(sel_ms) / len(sel_ms),
        "att_ms": sum(att_ms) / len(att_ms),
        "s4_ms": sum(s4_ms) / len(s4_ms),
        "s5_ms": sum(s5_ms) / len(s5_ms),
        "step_ms": sum(step_ms) / len(step_ms),
        "step_pct": pct(step_ms),
        "two_call_ms": sum(two_ms) / len(two_ms),
        "two_call_pct": pct(two_ms),
        "graph_ms": graph_ms,
        "warm_step_ms": sum(warm_ms) / len(warm_ms),
        "wall_s": wall,
        "inputs": t,
    }


def run_adaptive(cfg, steps, warmup, t, ratio_min=0.10, ratio_max=0.20, margin=0.0,
                 flush_bytes=1 << 30):
    """The decode step with anchor-adaptive selection (kept fraction per (b, kv head) between
    ratio_min and ratio_max, set by the sink/local anchors' scores)."""
    import numpy as np
    import torch

    import long_context_block_summary_amd as bsa

    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to(t["q"]), to(t["k"]), to(t["v"])
    N, bs = cfg.seq_len, cfg.block_size
    summ, _ = bsa.build_block_summaries(k, N, bs)
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    kw = dict(adaptive=True, keep_ratio_max=ratio_max, anchor_margin=margin)
    ts, kept = [], None
    for i in range(warmup + steps):
        flush.add_(1.0)
        e0, e1 = ev(), ev()
        e0.record(stream)
        out, lse, idx = bsa.decode_step(q, k, v, summ, N, bs, cfg.n_sink, cfg.n_local, -1,
                                        ratio_min, **kw)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            ts.append(e0.elapsed_time(e1))
        kept = (idx >= 0).sum(dim=2).float()
    ms = sum(ts) / len(ts)
    nb = -(-N // bs)
    return {"workload": cfg.name, "ms_per_step": ms,
            "queries_heads_per_s": cfg.batch * cfg.n_q_heads / (ms / 1e3), **pct(ts),
            "keep_range": [ratio_min, ratio_max], "anchor_margin": margin,
            "kept_pct_mean": float(kept.mean()) / nb * 100,
            "kept_pct_min": float(kept.min()) / nb * 100,
            "kept_pct_max": float(kept.max()) / nb * 100,
            "timed": "select_blocks (adaptive) + sparse_decode_attn, cold cache"}


def run_fp8(cfg, steps, warmup, t, flush_bytes=1 << 30):
    """The decode step over an FP8 (E4M3) copy of the cache: select_blocks (bf16 summaries) +
    sparse_decode_attn_fp8.  The quantization runs once at ingest and is timed on its own."""
    import numpy as np
    import torch

    import long_context_block_summary_amd as bsa

    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to(t["q"]), to(t["k"]), to(t["v"])
    N, bs = cfg.seq_len, cfg.block_size
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    summ, _ = bsa.build_block_summaries(k, N, bs)
    e0, e1 = ev(), ev()
    e0.record(stream)
    k8, ks = bsa.quantize_kv_fp8(k, N, bs)
    v8, vs = bsa.quantize_kv_fp8(v, N, bs)
    e1.record(stream)
    torch.cuda.synchronize()
    quant_ms = e0.elapsed_time(e1)
    del k, v
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    idx, _ = bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k, cfg.keep_ratio)
    n_keep = idx.shape[2]
    ws = torch.empty(max(16, bsa.decode_workspace_size(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads,
                                                       cfg.head_dim, N, n_keep)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.batch, cfg.n_q_heads), dtype=torch.float32, device=dev)
    step_ms, att_ms = [], []
    for i in range(warmup + steps):
        flush.add_(1.0)
        a, b_, c = ev(), ev(), ev()
        a.record(stream)
        bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k, cfg.keep_ratio,
                          block_idx=idx)
        b_.record(stream)
        bsa.sparse_decode_attn_fp8(q, k8, v8, ks, vs, idx, N, bs, out=out, lse=lse, workspace=ws)
        c.record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            step_ms.append(a.elapsed_time(c))
            att_ms.append(b_.elapsed_time(c))
    B, Hq, Hkv, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    kept_tokens = min(n_keep * bs, N)
    att_bytes = (B * Hkv * kept_tokens * d * 2 + B * Hkv * n_keep * 2 * 4 + B * Hq * d * 2
                 + B * Hq * d * 4 + B * Hkv * n_keep * 4)
    ms, am = sum(step_ms) / len(step_ms), sum(att_ms) / len(att_ms)
    return {"workload": cfg.name, "ms_per_step": ms,
            "queries_heads_per_s": B * Hq / (ms / 1e3), **pct(step_ms),
            "sparse_decode_attn_fp8_us": am * 1e3,
            "attn_algorithmic_bytes": att_bytes,
            "attn_GBps": att_bytes / (am / 1e3) / 1e9,
            "attn_frac_of_8TBps": att_bytes / (am / 1e3) / 1e9 / HBM_PEAK_GBS,
            "quantize_kv_ms_ingest": quant_ms,
            "format": "OCP E4M3 codes, one fp32 scale per (b, kv head, 64-token block) for K and V",
            "timed": "select_blocks + sparse_decode_attn_fp8, cold cache"}


def run_bf16_summaries(cfg, steps, warmup, t, flush_bytes=1 << 30):
    """The decode step on bf16 block summaries (half the bytes the scores read): select_blocks
    alone, select + attend as two calls, and the fused sparse_decode_step, cold cache."""
    import numpy as np
    import torch

    import long_context_block_summary_amd as bsa

    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to(t["q"]), to(t["k"]), to(t["v"])
    N, bs = cfg.seq_len, cfg.block_size
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    _, s16 = bsa.build_block_summaries(k, N, bs, want_f32=False, want_bf16=True)
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    sel = dict(n_sink=cfg.n_sink, n_local=cfg.n_local, top_k=cfg.top_k,
               keep_ratio=cfg.keep_ratio)
    idx, _ = bsa.select_blocks(q, s16, N, bs, **sel)
    out, lse = bsa.sparse_decode_attn(q, k, v, idx, N, bs)
    ws_sel = torch.empty(16 << 20, dtype=torch.uint8, device=dev)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    calls = {
        "select_blocks": lambda: bsa.select_blocks(q, s16, N, bs, block_idx=idx,
                                                   workspace=ws_sel, **sel),
        "step": lambda: (bsa.select_blocks(q, s16, N, bs, block_idx=idx, workspace=ws_sel, **sel),
                         bsa.sparse_decode_attn(q, k, v, idx, N, bs, out=out, lse=lse,
                                                workspace=ws)),
        "fused_step": lambda: bsa.sparse_decode_step(q, k, v, s16, N, bs, block_idx=idx, out=out,
                                                     lse=lse, workspace=ws, **sel),
    }
    res = {"workload": cfg.name,
           "summary_bytes": cfg.batch * cfg.n_kv_heads * (-(-N // bs)) * cfg.head_dim * 2}
    for name, fn in calls.items():
        ts = []
        for i in range(warmup + steps):
            flush.add_(1.0)
            a, c = ev(), ev()
            a.record(stream)
            fn()
            c.record(stream)
            torch.cuda.synchronize()
            if i >= warmup:
                ts.append(a.elapsed_time(c) * 1e3)
        res[name + "_us"] = sum(ts) / len(ts)
    res["queries_heads_per_s"] = cfg.batch * cfg.n_q_heads / (res["fused_step_us"] / 1e6)
    res["timed"] = "bf16 summaries (bsa_select_cfg.summaries_bf16), cold cache"
    return res


def run_decode_loop(cfg, steps, warmup, t, flush_bytes=1 << 30):
    """Per generated token: append K/V, refresh the summary of its block, select, attend.
    The cache holds the workload's tokens; the loop starts `warmup + steps` tokens before
    the end and appends the held tokens one by one (each step reads a cold cache)."""
    import numpy as np
    import torch

    import long_context_block_summary_amd as bsa

    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to(t["q"]), to(t["k"]), to(t["v"])
    N, bs = cfg.seq_len, cfg.block_size
    n0 = N - warmup - steps
    S = -(-N // bs)
    summ, _ = bsa.build_block_summaries(k, n0, bs, summary_stride=S)
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    ts = []
    for i in range(warmup + steps):
        n = n0 + i
        k_new = k[:, :, n:n + 1].contiguous()
        v_new = v[:, :, n:n + 1].contiguous()
        flush.add_(1.0)
        e0, e1 = ev(), ev()
        e0.record(stream)
        bsa.decode_loop_step(q, k_new, v_new, k, v, summ, n, bs, cfg.n_sink, cfg.n_local,
                             cfg.top_k, cfg.keep_ratio)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= warmup:
            ts.append(e0.elapsed_time(e1))
    ms = sum(ts) / len(ts)
    return {"workload": cfg.name, "ms_per_token": ms,
            "queries_heads_per_s": cfg.batch * cfg.n_q_heads / (ms / 1e3), **pct(ts),
            "timed": "decode_loop_step: append_kv (with the summary refresh) + "
                     "sparse_decode_step per generated token, cold cache, "
                     f"context {n0 + warmup}..{N}"}


def pct(xs):
    """p10 / median / p90 of a list of times."""
    s = sorted(xs)
    at = lambda f: s[min(len(s) - 1, int(round(f * (len(s) - 1))))]
    return {"p10": at(0.1), "median": at(0.5), "p90": at(0.9)}


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """Plain device-to-device copy of nbytes (read + write) as a measured ceiling, GB/s."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = sorted(ts)[len(ts) // 2]
    del a, b
    return {"bytes_moved": 2 * nbytes, "median_ms": ms, "GBps": 2 * nbytes / (ms / 1e3) / 1e9,
            "what": "torch copy_ of 1 GiB fp32 (read + write), median of 10"}


def prefill_flops(cfg, ksel, n_dense):
    """Algorithmic flops of the three attention branches (QK^T and PV, 2 flops per MAC)."""
    return 4 * cfg.head_dim * cfg.chunk_len * cfg.batch * cfg.n_q_heads * (ksel + n_dense + cfg.window)


def run_prefill(cfg, steps, warmup, flush_bytes=1 << 30):
    import numpy as np
    import torch

    import long_context_block_summary_amd as bsa
    from long_context_block_summary_amd import synth

    dev = torch.device("cuda:0")
    t = synth.gen_prefill(cfg)
    to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = to(t["q"]), to(t["k"]), to(t["v"])
    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    pc = bsa.prefill_cfg(cfg.m_sparse, cfg.top_k_sparse, cfg.m_dense, cfg.window, cfg.q_tile)
    r1 = []
    for _ in range(3):
        flush.add_(1.0)
        e0, e1 = ev(), ev()
        e0.record(stream)
        streams = bsa.build_compressed_streams(k, v, cfg.prior_len, pc)
        e1.record(stream)
        torch.cuda.synchronize()
        r1.append(e0.elapsed_time(e1))
    out = torch.empty((cfg.batch, cfg.chunk_len, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32,
                      device=dev)
    import ctypes
    shape = bsa.make_shape(cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.prior_len,
                           k.shape[2])
    ws = torch.empty(bsa.lib().bsa_prefill_workspace_size(ctypes.byref(shape), cfg.chunk_len,
                                                          ctypes.byref(pc)),
                     dtype=torch.uint8, device=dev)
    pc_cat = bsa.prefill_cfg(cfg.m_sparse, cfg.top_k_sparse, cfg.m_dense, cfg.window, cfg.q_tile,
                             bsa.COMBINE_CONCAT)
    # the selection against the fp32 means (the other indexer), reported beside the default
    pc_f32 = bsa.prefill_cfg(cfg.m_sparse, cfg.top_k_sparse, cfg.m_dense, cfg.window, cfg.q_tile,
                             indexer=bsa.INDEXER_F32)
    k4f, _ = bsa.build_block_summaries(k, cfg.prior_len, cfg.m_sparse, want_f32=True)
    sink = torch.linspace(-2.0, 3.0, cfg.n_q_heads, dtype=torch.float32, device=dev)
    sel = torch.empty((cfg.batch, -(-cfg.chunk_len // cfg.q_tile), cfg.n_kv_heads,
                       min(cfg.top_k_sparse, -(-cfg.prior_len // cfg.m_sparse))),
                      dtype=torch.int32, device=dev)
    calls = {
        "sparse_prefill_attn": lambda: bsa.sparse_prefill_attn(
            q, k, v, *streams, cfg.prior_len, cfg=pc, out=out, workspace=ws),
        "select_prefill_entries": lambda: bsa.select_prefill_entries(
            q, k, None, streams[1], cfg.prior_len, cfg=pc, sel=sel, workspace=ws),
        "select_prefill_entries_f32": lambda: bsa.select_prefill_entries(
            q, k, k4f, None, cfg.prior_len, cfg=pc_f32, sel=sel, workspace=ws),
        "sparse_prefill_attn_selected": lambda: bsa.sparse_prefill_attn_selected(
            q, k, v, *streams[1:], sel, cfg.prior_len, cfg=pc, out=out),
        "concat_sink": lambda: bsa.sparse_prefill_attn_selected(
            q, k, v, *streams[1:], sel, cfg.prior_len, cfg=pc_cat, out=out, sink_logits=sink),
    }
    times = {}
    for name, fn in calls.items():
        for _ in range(warmup):
            flush.add_(1.0)
            fn()
        ts = []
        for _ in range(steps):
            flush.add_(1.0)
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        times[name] = ts
    e4 = -(-cfg.prior_len // cfg.m_sparse)
    e128 = -(-cfg.prior_len // cfg.m_dense)
    ksel = min(cfg.top_k_sparse, e4)
    fl = prefill_flops(cfg, ksel, e128)
    mean = lambda xs: sum(xs) / len(xs)
    ms = mean(times["sparse_prefill_attn"])
    att = mean(times["sparse_prefill_attn_selected"])
    r2 = mean(times["select_prefill_entries"])
    n_tiles = -(-cfg.chunk_len // cfg.q_tile)
    # the bf16 keys read once, the fp32 scores written once and read back by the top-k
    r2_bytes = (cfg.batch * cfg.n_kv_heads * e4 * cfg.head_dim * 2
                + 2 * cfg.batch * cfg.n_kv_heads * n_tiles * e4 * 4)
    r2_flops = 2 * cfg.batch * cfg.n_kv_heads * n_tiles * e4 * cfg.head_dim
    r2_f32 = mean(times["select_prefill_entries_f32"])
    gather_a = cfg.batch * cfg.n_kv_heads * n_tiles * ksel * cfg.head_dim * 2 * 2
    return {"workload": cfg.name, "ms_per_call": ms, "call_pct": pct(times["sparse_prefill_attn"]),
            "algorithmic_gflop": fl / 1e9,
            "achieved_tflops": fl / (ms / 1e3) / 1e12,
            "frac_of_bf16_mfma_peak": fl / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "timed": "sparse_prefill_attn call: pooled queries + scores + top-k + 3-branch attention",
            "attention_R3_R6": {"call": "sparse_prefill_attn_selected", "ms": att,
                                "achieved_tflops": fl / (att / 1e3) / 1e12,
                                "frac_of_bf16_mfma_peak": fl / (att / 1e3) / 1e12
                                / MFMA_BF16_PEAK_TFLOPS,
                                "branch_A_gather_GBps_over_call": gather_a / (att / 1e3) / 1e9},
            "attention_concat_sink": {"call": "sparse_prefill_attn_selected, concatenated "
                                              "softmax + per-head sink logits",
                                      "ms": mean(times["concat_sink"])},
            "selection_R2": {"call": "select_prefill_entries (bf16 compressed keys)", "ms": r2,
                             "GBps": r2_bytes / (r2 / 1e3) / 1e9,
                             "bytes": r2_bytes, "gflop": r2_flops / 1e9,
                             "fp32_means_indexer_ms": r2_f32},
            "streams_ingest_ms": sorted(r1)[1], "inputs": t}


def run_cpu_baseline(cfg, t, budget_s=20.0, min_s=10.0, one_thread_s=4.0, others=None):
    """Oracle select + attend (given its fp64 summaries) on a bounded sample, on every host
    thread and on one; the oracle's summaries alone; and one-thread select + attend on other
    decode workloads (`others`: name -> (config, inputs))."""
    import oracle
    B = cfg.batch
    t0 = time.perf_counter()
    summ = oracle.block_summaries(t["k"], cfg.seq_len, cfg.block_size)
    summ_s = time.perf_counter() - t0

    def one(c, inp, sm, bsl):
        t0 = time.perf_counter()
        idx, _ = oracle.select_blocks(inp["q"][bsl], sm[bsl], c.n_kv_heads, c.n_sink,
                                      c.n_local, c.top_k, c.keep_ratio)
        oracle.sparse_decode_attn(inp["q"][bsl], inp["k"][bsl], inp["v"][bsl], idx, c.seq_len,
                                  c.block_size)
        return time.perf_counter() - t0

    first = one(cfg, t, summ, slice(0, 1))
    nb_used = 1
    if first * B <= budget_s and B > 1:
        nb_used = B
    # repeat the pass until about min_s of CPU time has been spent (bounded by budget_s)
    reps, elapsed = 0, 0.0
    while reps == 0 or (elapsed < min_s and elapsed + elapsed / reps <= budget_s):
        elapsed += one(cfg, t, summ, slice(0, nb_used))
        reps += 1
    qh = reps * nb_used * cfg.n_q_heads
    cores = oracle.num_threads()
    k_bytes = cfg.batch * cfg.n_kv_heads * cfg.seq_len * cfg.head_dim * 2

    def one_thread(c, inp, sm, limit_s):
        reps1, el1 = 0, 0.0
        while reps1 == 0 or el1 < limit_s:
            el1 += one(c, inp, sm, slice(0, 1))
            reps1 += 1
        return {"value": reps1 * c.n_q_heads / el1, "unit": "queries*heads/s",
                "sample": f"{c.name}: 1 of {c.batch} batch entries, {reps1} passes, {el1:.2f} s"}

    # the same oracle on one thread, over one batch entry (bounded to a few seconds each)
    others = others or {}
    other_summ = {name: oracle.block_summaries(inp["k"], c.seq_len, c.block_size)
                  for name, (c, inp) in others.items()}
    oracle.set_threads(1)
    try:
        one_t = one_thread(cfg, t, summ, one_thread_s)
        one_t_others = {name: one_thread(c, inp, other_summ[name], one_thread_s / 2)
                        for name, (c, inp) in others.items()}
    finally:
        oracle.set_threads(cores)
    return {"value": qh / elapsed, "unit": "queries*heads/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{cfg.name}: select + attend (fp64 oracle, summaries precomputed) for "
                      f"{nb_used} of {B} batch entries ({nb_used * cfg.n_q_heads} query heads), "
                      f"{reps} passes, {elapsed:.2f} s",
            "one_thread": one_t,
            "one_thread_other_workloads": one_t_others,
            "summaries_alone": {"s": summ_s, "key_GBps": k_bytes / summ_s / 1e9, "cores": cores,
                                "sample": f"{cfg.name}: fp64 means of every 64-token block of "
                                          f"K ({k_bytes / 1e9:.2f} GB of bf16 keys), once"},
            "host": host_description()}


def run_cpu_prefill_baseline(cfg, t, big_tiles=4):
    """The oracle's prefill on sampled query rows.  Its call builds the compressed streams from
    the raw cache every time (a fixed cost), so the select + attend rate given the streams is
    taken as the difference between a call over `big_tiles` whole tiles and a call over one
    tile; the streams alone (fp64 means, no rounding) and the whole larger call are reported
    beside it."""
    import numpy as np

    import oracle
    P = cfg.prior_len
    common = dict(m_sparse=cfg.m_sparse, top_k=cfg.top_k_sparse, m_dense=cfg.m_dense,
                  window=cfg.window, q_tile=cfg.q_tile)
    rows_small = np.arange(cfg.q_tile, dtype=np.int32)
    rows_big = np.arange(big_tiles * cfg.q_tile, dtype=np.int32)
    t0 = time.perf_counter()
    for x in (t["k"], t["v"]):
        for m in (cfg.m_sparse, cfg.m_dense):
            oracle.block_summaries(x, P, m)
    streams_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.sparse_prefill_attn(t["q"], t["k"], t["v"], P, rows=rows_small, **common)
    small_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.sparse_prefill_attn(t["q"], t["k"], t["v"], P, rows=rows_big, **common)
    big_s = time.perf_counter() - t0
    e4 = -(-P // cfg.m_sparse)
    n_ent = min(cfg.top_k_sparse, e4) + -(-P // cfg.m_dense) + cfg.window
    d_rows = len(rows_big) - len(rows_small)
    marg = max(big_s - small_s, 1e-9)
    qh = d_rows * cfg.n_q_heads
    return {"value": qh / marg, "unit": "queries*heads/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "gflops_fp64": 4 * cfg.head_dim * n_ent * qh / marg / 1e9,
            "sample": f"{cfg.name}: oracle calls over {len(rows_big)} and {len(rows_small)} "
                      f"query rows ({big_tiles} and 1 tiles, {cfg.n_q_heads} heads each) took "
                      f"{big_s:.2f} s and {small_s:.2f} s; the rate is the {d_rows} extra rows "
                      f"over the difference (both calls build the same streams)",
            "whole_call_s": big_s, "streams_alone_s": streams_s,
            "host": host_description()}


def host_description():
    """Logical CPUs and the CPU model of the host the oracle ran on."""
    model = None
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long128k_15")
    ap.add_argument("--also", default="long128k,gqa32k,ctx1m",
                    help="comma list of extra decode workloads reported alongside ('none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill", default="prefill256k",
                    help="prefill workload reported alongside ('none' to skip)")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None,
                    help="run only the prefill measurement, or only the decode step and its "
                         "FP8 line, and print their object (for counter passes); the default "
                         "runs the full bench")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path shards by (batch, kv head) with no exchange; see the design "
              "notes)", file=sys.stderr)
        sys.exit(2)

    from long_context_block_summary_amd import synth
    if args.only == "prefill":
        pr = run_prefill(synth.CONFIGS[args.prefill], args.steps, args.warmup)
        pr.pop("inputs")
        print(json.dumps(pr), flush=True)
        return
    cfg = synth.CONFIGS[args.workload]
    r = run_gpu(cfg, args.steps, args.warmup)
    if args.only == "decode":
        print(json.dumps({"workload": cfg.name, "ms_per_step": r["step_ms"],
                          "breakdown_us": {"select_blocks": r["sel_ms"] * 1e3,
                                           "sparse_decode_attn": r["att_ms"] * 1e3},
                          "fp8_kv": run_fp8(cfg, args.steps, args.warmup, r["inputs"])}),
              flush=True)
        return
    sel_b, att_b = decode_bytes(cfg, r["n_keep"])
    s4_b = partials_bytes(cfg, r["n_keep"])
    qh = cfg.batch * cfg.n_q_heads
    step_s = r["step_ms"] / 1e3
    att_gbs = att_b / (r["att_ms"] / 1e3) / 1e9
    s4_gbs = s4_b / (r["s4_ms"] / 1e3) / 1e9
    line = {
        "metric": METRIC,
        "value": qh / step_s,
        "unit": "queries*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "seq_len": cfg.seq_len, "block_size": cfg.block_size,
                   "n_sink_blocks": cfg.n_sink, "n_local_blocks": cfg.n_local,
                   "top_k": cfg.top_k, "n_keep": r["n_keep"],
                   "keep_pct": round(100.0 * r["n_keep"] / -(-cfg.seq_len // cfg.block_size), 2)},
        "step": "one sparse_decode_step call per step (block scores; the top-k inside the "
                "split-K attention launch where the candidates fit; the exact merge), 1 GiB "
                "cache flush before each",
        "two_call_step": {"calls": "select_blocks + sparse_decode_attn",
                          "ms_per_step": r["two_call_ms"],
                          "queries_heads_per_s": qh / (r["two_call_ms"] / 1e3),
                          **r["two_call_pct"]},
        "step_bytes": step_bytes(cfg, r["n_keep"]),
        "step_GBps": step_bytes(cfg, r["n_keep"]) / step_s / 1e9,
        "step_frac": step_bytes(cfg, r["n_keep"]) / step_s / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm",
                     "kernel": "decode_kernel (step S4, the sparse_decode_partials call)",
                     "achieved": s4_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": s4_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(cfg.name, "s4_traffic_bytes_per_launch"),
                     "algorithmic_bytes": s4_b, "avg_us": r["s4_ms"] * 1e3},
        "attention_call": {"call": "sparse_decode_attn (S4 + S5)", "avg_us": r["att_ms"] * 1e3,
                           "algorithmic_bytes": att_b, "GBps": att_gbs,
                           "frac": att_gbs / HBM_PEAK_GBS,
                           "traffic": measured_traffic(cfg.name)},
        "breakdown_us": {"select_blocks": r["sel_ms"] * 1e3,
                         "sparse_decode_attn": r["att_ms"] * 1e3,
                         "sparse_decode_partials": r["s4_ms"] * 1e3,
                         "sparse_decode_merge": r["s5_ms"] * 1e3,
                         "build_block_summaries_ingest": r["sum_ms"] * 1e3},
        "select_GBps": sel_b / (r["sel_ms"] / 1e3) / 1e9,
        "warm_cache_ms_per_step": r["warm_step_ms"],
        "step_ms_pct": r["step_pct"],
        "graph_step": (r["graph_ms"] if isinstance(r["graph_ms"], str) else
                       {"ms_per_step": sum(r["graph_ms"]) / len(r["graph_ms"]),
                        "queries_heads_per_s": qh / (sum(r["graph_ms"]) / len(r["graph_ms"]) / 1e3),
                        **pct(r["graph_ms"])}),
        "copy_ceiling": copy_bandwidth(),
        "timed_wall_s": r["wall_s"],
        "cache_flush": "1 GiB read+write before every step (untimed)",
    }
    extra, keep_inputs = {}, {}
    for name in [s for s in args.also.split(",") if s and s != "none"]:
        c2 = synth.CONFIGS[name]
        same = (c2.batch, c2.n_q_heads, c2.n_kv_heads, c2.head_dim, c2.seq_len) == \
            (cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len) and \
            synth.DEFAULT_SEED.get(name) == synth.DEFAULT_SEED.get(cfg.name)
        r2 = run_gpu(c2, max(10, args.steps // 2), 3, inputs=r["inputs"] if same else None)
        _, a2 = decode_bytes(c2, r2["n_keep"])
        st2 = step_bytes(c2, r2["n_keep"])
        p2 = partials_bytes(c2, r2["n_keep"])
        extra[name] = {"queries_heads_per_s": c2.batch * c2.n_q_heads / (r2["step_ms"] / 1e3),
                       "ms_per_step": r2["step_ms"], "n_keep": r2["n_keep"],
                       "step_bytes": st2,
                       "step_GBps": st2 / (r2["step_ms"] / 1e3) / 1e9,
                       "step_frac": st2 / (r2["step_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                       "attn_GBps": a2 / (r2["att_ms"] / 1e3) / 1e9,
                       "attn_frac": a2 / (r2["att_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                       "s4_us": r2["s4_ms"] * 1e3,
                       "s4_frac": p2 / (r2["s4_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS,
                       "select_us": r2["sel_ms"] * 1e3, "attn_us": r2["att_ms"] * 1e3}
        if name == "ctx1m":
            extra[name]["bf16_summaries"] = run_bf16_summaries(c2, max(10, args.steps // 2), 3,
                                                               r2["inputs"])
        if name in ("tiny", "gqa32k", "long128k"):
            keep_inputs[name] = (c2, r2["inputs"])
        del r2
    line["bf16_summaries"] = run_bf16_summaries(cfg, max(10, args.steps // 2), 3, r["inputs"])
    line["decode_loop"] = run_decode_loop(cfg, max(10, args.steps // 2), 3, r["inputs"])
    line["adaptive_selection"] = run_adaptive(cfg, max(10, args.steps // 2), 3, r["inputs"])
    line["fp8_kv"] = run_fp8(cfg, max(10, args.steps // 2), 3, r["inputs"])
    pf_inputs = None
    if args.prefill and args.prefill != "none":
        line["prefill"] = run_prefill(synth.CONFIGS[args.prefill], max(5, args.steps // 5), 2)
        pf_inputs = line["prefill"].pop("inputs")
    if extra:
        line["also"] = extra
    if not args.no_cpu_baseline:
        if "tiny" not in keep_inputs:
            keep_inputs["tiny"] = (synth.CONFIGS["tiny"], synth.gen_decode(synth.CONFIGS["tiny"]))
        line["cpu_baseline"] = run_cpu_baseline(cfg, r["inputs"], others=keep_inputs)
        if pf_inputs is not None:
            line["cpu_baseline_prefill"] = run_cpu_prefill_baseline(
                synth.CONFIGS[args.prefill], pf_inputs)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
