"""GPU parity of the incremental decode loop: per generated token, append K/V,
refresh the summary of the block the token lands in (or opens), select, attend.

The incrementally kept summaries must equal a rebuild from scratch bit for bit;
selection and outputs must match the oracle run afresh on the whole cache at
every step.  Every case prints its name, seed and sizes before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import long_context_block_summary_amd as bsa
from long_context_block_summary_amd import synth
from parity_rules import OUT_ATOL, check_index_sets, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    bsa.lib()
    yield
    torch.cuda.synchronize()


def announce(*a):
    print("[case]", *a, flush=True)


def run_loop(name, seed, B, Hq, Hkv, d, n0, steps, capacity, top_k=-1, keep_ratio=0.0,
             check_every=1):
    import torch
    bs = 64
    announce(name, "seed", seed, "B", B, "Hq", Hq, "Hkv", Hkv, "d", d, "start", n0, "steps",
             steps, "capacity", capacity, "top_k", top_k, "keep_ratio", keep_ratio)
    cfg = synth.DecodeConfig(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                             seq_len=n0 + steps, top_k=top_k, keep_ratio=keep_ratio)
    t = synth.gen_decode(cfg, seed, capacity=capacity)
    rng = np.random.default_rng(seed + 1000)
    dev = torch.device("cuda:0")
    k_all, v_all = to_dev(t["k"]), to_dev(t["v"])
    k_cache = torch.zeros_like(k_all)
    v_cache = torch.zeros_like(v_all)
    k_cache[:, :, :n0] = k_all[:, :, :n0]
    v_cache[:, :, :n0] = v_all[:, :, :n0]
    S = -(-capacity // bs)
    summ, _ = bsa.build_block_summaries(k_cache, n0, bs, summary_stride=S)
    k_host = t["k"].copy()
    k_host[:, :, n0:] = 0
    v_host = t["v"].copy()
    v_host[:, :, n0:] = 0
    worst, exempt_total = 0.0, 0
    for s in range(steps):
        N = n0 + s
        q16 = synth.bf16_round(rng.standard_normal((B, Hq, d)).astype(np.float32))
        q = to_dev(q16)
        k_new = k_all[:, :, N:N + 1].contiguous()
        v_new = v_all[:, :, N:N + 1].contiguous()
        out, lse, idx = bsa.decode_loop_step(q, k_new, v_new, k_cache, v_cache, summ, N, bs,
                                             top_k=top_k, keep_ratio=keep_ratio)
        k_host[:, :, N] = t["k"][:, :, N]
        v_host[:, :, N] = t["v"][:, :, N]
        if s % check_every and s != steps - 1:
            continue
        torch.cuda.synchronize()
        n1 = N + 1
        nb = -(-n1 // bs)
        # the incremental summaries equal a rebuild of the whole cache, bit for bit
        fresh, _ = bsa.build_block_summaries(k_cache, n1, bs)
        assert torch.equal(summ[:, :, :nb], fresh), f"step {s}: incremental summaries differ"
        # and the oracle's fp32 token-order means, bit for bit
        assert np.array_equal(summ[:, :, :nb].cpu().numpy(),
                              oracle.block_summaries_f32(k_host, n1, bs)), \
            f"step {s}: summaries differ from the oracle's"
        # the cache holds exactly the appended tokens
        assert torch.equal(k_cache[:, :, :n1], k_all[:, :, :n1])
        assert torch.equal(v_cache[:, :, :n1], v_all[:, :, :n1])
        # selection and output against the oracle on the whole cache, from scratch
        o_summ = oracle.block_summaries(k_host, n1, bs)
        o_idx, o_scores = oracle.select_blocks(q16, o_summ, Hkv, 1, 2, top_k, keep_ratio)
        g_idx = idx.cpu().numpy()
        exempt_total += check_index_sets(g_idx, o_idx, o_scores, nb, 1, 2)
        o_out, o_lse, _ = oracle.sparse_decode_attn(q16, k_host, v_host, g_idx, n1, bs)
        err = float(np.abs(out.cpu().numpy() - o_out).max())
        lerr = float(np.abs(lse.cpu().numpy() - o_lse).max())
        assert err <= OUT_ATOL and lerr <= 1e-3, (s, err, lerr)
        worst = max(worst, err)
    announce("  worst |out err|", worst, "exempt ties", exempt_total)


def test_loop_crosses_block_boundaries():
    # starts 4 tokens before a block boundary; 70 tokens open two more blocks
    run_loop("loop_g4", 41, B=2, Hq=8, Hkv=2, d=128, n0=64 * 12 + 60, steps=70,
             capacity=64 * 16, top_k=5)


def test_loop_keep_ratio_group8_d64():
    # keep ratio: the number of kept blocks grows as blocks open
    run_loop("loop_ratio", 42, B=1, Hq=8, Hkv=1, d=64, n0=64 * 9 + 1, steps=130,
             capacity=64 * 12, keep_ratio=0.3, check_every=7)


def test_loop_from_an_empty_block():
    # the cache starts at an exact block boundary and at a single token
    run_loop("loop_edge", 43, B=1, Hq=4, Hkv=4, d=128, n0=64 * 3, steps=3, capacity=64 * 5,
             top_k=1)
    run_loop("loop_one", 44, B=1, Hq=4, Hkv=2, d=128, n0=1, steps=66, capacity=64 * 3, top_k=2,
             check_every=5)


@pytest.mark.parametrize("bs,n_new", [(64, 150), (128, 5), (256, 300), (16, 1)])
def test_append_refresh_matches_rebuild(bs, n_new):
    # several tokens per append (several blocks refreshed in one launch), other block sizes
    # (256 takes the separate append + refresh path), and d = 64
    import torch
    B, H, d, cap, n0 = 2, 3, 64, 1200, 333
    announce("append_refresh", "bs", bs, "n_new", n_new, "B", B, "H", H, "d", d, "start", n0)
    rng = np.random.default_rng(bs + n_new)
    kv = synth.bf16_round(rng.standard_normal((2, B, H, cap, d)).astype(np.float32))
    k_all, v_all = to_dev(kv[0]), to_dev(kv[1])
    k_cache, v_cache = torch.zeros_like(k_all), torch.zeros_like(v_all)
    k_cache[:, :, :n0] = k_all[:, :, :n0]
    v_cache[:, :, :n0] = v_all[:, :, :n0]
    S = -(-cap // bs)
    summ, _ = bsa.build_block_summaries(k_cache, n0, bs, summary_stride=S)
    n = n0
    while n + n_new <= cap:
        bsa.append_kv(k_all[:, :, n:n + n_new].contiguous(), v_all[:, :, n:n + n_new].contiguous(),
                      k_cache, v_cache, n, bs, summ)
        n += n_new
        if n > n0 + 4 * n_new:
            break
    torch.cuda.synchronize()
    nb = -(-n // bs)
    fresh, _ = bsa.build_block_summaries(k_cache, n, bs)
    assert torch.equal(summ[:, :, :nb], fresh)
    assert torch.equal(k_cache[:, :, :n], k_all[:, :, :n])
    assert torch.equal(v_cache[:, :, :n], v_all[:, :, :n])
    assert not k_cache[:, :, n:].any() and not v_cache[:, :, n:].any()
    # appending without a summaries buffer only writes the rows
    m = min(7, cap - n)
    bsa.append_kv(k_all[:, :, n:n + m].contiguous(), v_all[:, :, n:n + m].contiguous(), k_cache,
                  v_cache, n)
    torch.cuda.synchronize()
    assert torch.equal(k_cache[:, :, :n + m], k_all[:, :, :n + m])
    assert torch.equal(summ[:, :, :nb], fresh)


def test_loop_at_the_128k_workload_shape():
    # the 128K / 15 % workload's shapes, 10 tokens before the end of its last full block:
    # the loop fills that block and opens the next one
    run_loop("loop_128k", 45, B=4, Hq=64, Hkv=8, d=128, n0=131062, steps=14,
             capacity=131072 + 64, top_k=304)
