"""Randomised GPU parity of the decode path against the oracle.

32 seeded cases draw the batch, kv heads, group size, head dim, length
(log-uniform from 1 to 24,000 tokens), sink/local counts, top-k or keep ratio,
split count and the data (planted block strengths or plain Gaussian); each case
runs the summaries, the selection and the attention on the GPU and checks them
against the oracle as the fixed-shape tests do (fp32 summaries bit for bit, index
sets by the near-tie rule, outputs within 2e-3), then requires the fused step to
give the same list and outputs bit for bit.  16 more draws run the FP8 cache:
the GPU quantizer against the oracle's codes and scales bit for bit, then the FP8
attention (a quarter of them over adaptive, -1-padded lists) within 2e-3.  16
random anchor-adaptive selections are checked against the oracle's rule, 8 random
decode loops step by step, and 8 long-context cases (20,000 to 200,000 tokens).
Every case prints its parameters before any GPU call.
"""
import math

import numpy as np
import pytest

import long_context_block_summary_amd as bsa
from long_context_block_summary_amd import synth
from parity_rules import to_dev
from test_gpu_decode import announce, run_decode_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    bsa.lib()
    yield
    torch.cuda.synchronize()


def draw_case(i):
    rng = np.random.default_rng(7000 + i)
    g = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4]))
    n_sink, n_local = int(rng.integers(0, 4)), int(rng.integers(0, 4))
    ratio = bool(rng.integers(0, 2))
    top_k = -1 if ratio else int(rng.integers(0, 120))
    keep = float(rng.choice([0.05, 0.1, 0.15, 0.2, 0.35])) if ratio else 0.0
    if n_sink + n_local == 0 and (ratio or top_k == 0):
        n_local = 1  # at least one kept block per list
    cfg = synth.DecodeConfig(
        name=f"rand{i}", batch=int(rng.integers(1, 4)), n_q_heads=hkv * g, n_kv_heads=hkv,
        head_dim=int(rng.choice([64, 128])),
        seq_len=int(math.exp(rng.uniform(0.0, math.log(24000)))),
        n_sink=n_sink, n_local=n_local, top_k=top_k, keep_ratio=keep,
        planted=bool(rng.integers(0, 2)))
    return cfg, int(rng.choice([0, 1, 3, 8])), int(rng.integers(0, 10**6))


@pytest.mark.parametrize("i", range(32))
def test_random_decode_shapes(i):
    import torch
    cfg, n_splits, seed = draw_case(i)
    run_decode_case(cfg, seed, n_splits=n_splits)
    # the fused step: the same list and, bit for bit, the same outputs
    announce("  fused step", cfg.name)
    t = synth.gen_decode(cfg, seed)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    N, bs = cfg.seq_len, cfg.block_size
    summ, _ = bsa.build_block_summaries(k, N, bs)
    idx, _ = bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k,
                               cfg.keep_ratio)
    out, lse = bsa.sparse_decode_attn(q, k, v, idx, N, bs)
    out2, lse2, idx2 = bsa.sparse_decode_step(q, k, v, summ, N, bs, cfg.n_sink, cfg.n_local,
                                              cfg.top_k, cfg.keep_ratio)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx)
    assert torch.equal(out2, out) and torch.equal(lse2, lse)


@pytest.mark.parametrize("i", range(16))
def test_random_fp8_decode_shapes(i):
    """The same draws over an FP8 (E4M3) cache: quantize_kv_fp8 writes the oracle's codes
    and scales bit for bit, and sparse_decode_attn_fp8 on the GPU's selection matches the
    oracle's attention over the dequantized cache (within 2e-3), with or without an
    adaptive selection's -1 padding."""
    import torch
    import oracle
    from parity_rules import OUT_ATOL
    cfg, _, seed = draw_case(100 + i)
    adaptive = i % 4 == 3
    announce(cfg.name, "fp8 seed", seed, "B", cfg.batch, "Hq", cfg.n_q_heads, "Hkv",
             cfg.n_kv_heads, "d", cfg.head_dim, "N", cfg.seq_len, "sink", cfg.n_sink, "local",
             cfg.n_local, "top_k", cfg.top_k, "ratio", cfg.keep_ratio, "adaptive", adaptive)
    t = synth.gen_decode(cfg, seed)
    N, bs = cfg.seq_len, cfg.block_size
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    k8, ks = bsa.quantize_kv_fp8(k, N, bs)
    v8, vs = bsa.quantize_kv_fp8(v, N, bs)
    summ, _ = bsa.build_block_summaries(k, N, bs)
    kw = dict(adaptive=True, keep_ratio_max=0.3) if adaptive else {}
    idx, _ = bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k,
                               0.1 if adaptive else cfg.keep_ratio, **kw)
    out, lse = bsa.sparse_decode_attn_fp8(q, k8, v8, ks, vs, idx, N, bs)
    torch.cuda.synchronize()
    nb = -(-N // bs)
    o_k8, o_ks = oracle.quantize_fp8(t["k"], N, bs)
    o_v8, o_vs = oracle.quantize_fp8(t["v"], N, bs)
    assert np.array_equal(k8.cpu().numpy()[:, :, :N], o_k8[:, :, :N])
    assert np.array_equal(v8.cpu().numpy()[:, :, :N], o_v8[:, :, :N])
    assert np.array_equal(ks.cpu().numpy()[..., :nb].view(np.uint32), o_ks[..., :nb].view(np.uint32))
    assert np.array_equal(vs.cpu().numpy()[..., :nb].view(np.uint32), o_vs[..., :nb].view(np.uint32))
    o_out, o_lse = oracle.sparse_decode_attn_fp8(t["q"], o_k8, o_v8, o_ks, o_vs,
                                                 idx.cpu().numpy(), N, bs)
    err = float(np.abs(out.cpu().numpy() - o_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - o_lse).max())
    announce("  max|out err|", err, "max|lse err|", lerr)
    assert err <= OUT_ATOL and lerr <= 1e-3


@pytest.mark.parametrize("i", range(16))
def test_random_adaptive_shapes(i):
    """Seeded random anchor-adaptive selections (keep range, anchor margin, batch, heads,
    head dim, 261 to 40,000 tokens) against the oracle's adaptive rule, and the attention
    over the -1-padded lists (the checks of test_gpu_adaptive.run_adaptive)."""
    from test_gpu_adaptive import run_adaptive
    rng = np.random.default_rng(8000 + i)
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    rmin = float(rng.choice([0.05, 0.1, 0.15]))
    rmax = rmin + float(rng.choice([0.05, 0.1, 0.2]))
    margin = float(rng.choice([0.0, rng.uniform(-1.0, 1.0)]))
    N = int(math.exp(rng.uniform(math.log(64 * 4 + 5), math.log(40000))))
    run_adaptive(f"rand_adapt{i}", int(rng.integers(0, 10**6)), B=int(rng.integers(1, 4)),
                 Hq=hkv * g, Hkv=hkv, d=int(rng.choice([64, 128])), N=N, rmin=rmin, rmax=rmax,
                 margin=margin)


@pytest.mark.parametrize("i", range(8))
def test_random_decode_loop_shapes(i):
    """Seeded random decode loops (start length 1 to 6,000 tokens, 40-140 generated tokens,
    spare capacity, top-k or keep ratio): summaries equal a rebuild bit for bit and
    selection and outputs match the oracle afresh at every step (the checks of
    test_gpu_decode_loop.run_loop)."""
    from test_gpu_decode_loop import run_loop
    rng = np.random.default_rng(8500 + i)
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    n0 = int(rng.integers(1, 6001))
    steps = int(rng.integers(40, 141))
    ratio = bool(rng.integers(0, 2))
    run_loop(f"rand_loop{i}", int(rng.integers(0, 10**6)), B=int(rng.integers(1, 3)),
             Hq=hkv * g, Hkv=hkv, d=int(rng.choice([64, 128])), n0=n0, steps=steps,
             capacity=n0 + steps + int(rng.integers(0, 300)),
             top_k=-1 if ratio else int(rng.integers(1, 40)),
             keep_ratio=float(rng.choice([0.1, 0.2, 0.3])) if ratio else 0.0,
             check_every=max(1, steps // 20))


@pytest.mark.parametrize("i", range(8))
def test_random_long_decode_shapes(i):
    """Seeded random decode at long contexts (20,000 to 200,000 tokens log-uniform, 1-4 kv
    heads, groups 1-16, top-k up to 2,000 or a keep ratio, explicit split counts)."""
    rng = np.random.default_rng(77000 + i)
    g = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4]))
    ratio = bool(rng.integers(0, 2))
    cfg = synth.DecodeConfig(
        name=f"long_rand{i}", batch=int(rng.integers(1, 3)), n_q_heads=hkv * g, n_kv_heads=hkv,
        head_dim=int(rng.choice([64, 128])),
        seq_len=int(math.exp(rng.uniform(math.log(20000), math.log(200000)))),
        n_sink=int(rng.integers(0, 3)), n_local=int(rng.integers(1, 4)),
        top_k=-1 if ratio else int(rng.integers(1, 2000)),
        keep_ratio=float(rng.choice([0.05, 0.1, 0.15, 0.2])) if ratio else 0.0,
        planted=bool(rng.integers(0, 2)))
    run_decode_case(cfg, int(rng.integers(0, 10**6)), n_splits=int(rng.choice([0, 0, 2, 5])))
