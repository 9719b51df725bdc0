"""sparse_decode_step_noalloc (the decode step on the library's static scratch, for callers
that cannot allocate) against sparse_decode_step on the same inputs: the kept lists and
outputs must be bit-identical, on two calls in a row (the second one smaller, so it runs
on scratch the first call left behind), through the C ABI.

Every case prints its name and shapes before touching the GPU.
"""
import ctypes

import numpy as np
import pytest

import long_context_block_summary_amd as bsa
from long_context_block_summary_amd import synth
from parity_rules import to_dev

pytestmark = pytest.mark.gpu


def announce(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def L():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    lib = bsa.lib()
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.sparse_decode_step_noalloc.argtypes = [vp, vp, vp, vp, P(bsa.bsa_shape),
                                               P(bsa.bsa_select_cfg), vp, ctypes.c_float, vp, vp,
                                               vp]
    lib.sparse_decode_step_noalloc.restype = ctypes.c_int
    return lib


def _inputs(cfg, seed, bf16=False):
    t = synth.gen_decode(cfg, seed)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    s32, s16 = bsa.build_block_summaries(k, cfg.seq_len, 64, want_f32=not bf16, want_bf16=bf16)
    summ = s16 if bf16 else s32
    return q, k, v, summ


def _noalloc(L, q, k, v, summ, cfg):
    import torch
    B, Hq, d = q.shape
    Hkv, stride = k.shape[1], k.shape[2]
    nb = bsa.num_blocks(cfg.seq_len, 64)
    sc = bsa.select_cfg(64, cfg.n_sink, cfg.n_local, cfg.top_k, cfg.keep_ratio,
                        summaries_bf16=summ.dtype == torch.bfloat16)
    n_keep = bsa.num_kept(nb, sc)
    shape = bsa.make_shape(B, Hq, Hkv, d, cfg.seq_len, stride, summ.shape[2])
    idx = torch.full((B, Hkv, n_keep), -5, dtype=torch.int32, device=q.device)
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    rc = L.sparse_decode_step_noalloc(bsa._ptr(q), bsa._ptr(k), bsa._ptr(v), bsa._ptr(summ),
                                      ctypes.byref(shape), ctypes.byref(sc), bsa._ptr(idx), 0.0,
                                      bsa._ptr(out), bsa._ptr(lse), bsa._stream(q.device))
    assert rc == 0, rc
    return out, lse, idx


def _compare(L, cfg, seed, bf16=False):
    import torch
    announce(cfg.name, "seed", seed, "B", cfg.batch, "Hq", cfg.n_q_heads, "Hkv", cfg.n_kv_heads,
             "N", cfg.seq_len, "top_k", cfg.top_k, "keep_ratio", cfg.keep_ratio,
             "bf16 summaries", bf16)
    q, k, v, summ = _inputs(cfg, seed, bf16)
    o1, l1, i1 = _noalloc(L, q, k, v, summ, cfg)
    o2, l2, i2 = bsa.sparse_decode_step(q, k, v, summ, cfg.seq_len, 64, cfg.n_sink, cfg.n_local,
                                        cfg.top_k, cfg.keep_ratio)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.isfinite(o1).all()


def test_noalloc_step_equals_the_step_twice(L):
    # the 128K workload at 15 % (selection fused into the attention launch), then a smaller
    # ragged one with another group size on the scratch the first call left behind
    _compare(L, synth.CONFIGS["long128k_15"], 3)
    _compare(L, synth.DecodeConfig("noalloc_small", 2, 16, 4, 128, 64 * 90 + 17, top_k=9), 7)


def test_noalloc_step_unfused_selection_and_limit(L):
    # more than 4,096 candidates: the top-k runs as its own launch inside the step
    _compare(L, synth.DecodeConfig("noalloc_unfused", 1, 16, 2, 128, 64 * 5000, top_k=400), 8)
    _compare(L, synth.DecodeConfig("noalloc_keep_ratio", 1, 8, 8, 64, 64 * 40, keep_ratio=0.35),
             9)
    # on bf16 summaries, fused and unfused
    _compare(L, synth.DecodeConfig("noalloc_bf16", 2, 16, 4, 128, 64 * 90 + 17, top_k=9), 10,
             bf16=True)
    _compare(L, synth.DecodeConfig("noalloc_bf16_unfused", 1, 16, 2, 128, 64 * 5000, top_k=400),
             11, bf16=True)
    # a step whose workspace would exceed the static scratch is refused before any launch
    fake = ctypes.c_void_p(0x1000)
    big = bsa.make_shape(256, 64, 8, 128, 131072, 131072)
    cfg = bsa.select_cfg(top_k=304)
    assert L.bsa_decode_step_workspace_size(ctypes.byref(big), ctypes.byref(cfg)) > 16 << 20
    assert L.sparse_decode_step_noalloc(fake, fake, fake, fake, ctypes.byref(big),
                                        ctypes.byref(cfg), fake, 0.0, fake, None, None) == -2
