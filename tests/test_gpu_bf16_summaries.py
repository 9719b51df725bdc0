"""GPU parity of the decode path on bf16 block summaries (bsa_select_cfg.summaries_bf16):
the summaries are the bf16 rounding (ties to even) of the fp32 token-order means, and the
selection scores the pooled query against them.  The oracle runs its selection on the
same bf16 values (its fp32 token-order means, rounded), so both sides rank identical
keys: index sets by the near-tie rule, scores within the fp32 bound of the dot product,
attention within 2e-3 on the GPU's own index set; the fused step must agree with the two
calls bit for bit, and the decode loop's refreshed summaries with a rebuild.

Every case prints its name, seed and sizes before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import long_context_block_summary_amd as bsa
from long_context_block_summary_amd import synth
from parity_rules import OUT_ATOL, TIE_REL, check_index_sets, to_dev
from test_gpu_adaptive import oracle_topk
from test_gpu_decode import score_bound

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


def bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_bf16_summaries(k_u16, N, bs):
    """The oracle's fp32 token-order means rounded to bf16, as float64 [B][H][nb][d]."""
    rne = np.vectorize(oracle.round_bf16, otypes=[np.uint16])
    s32 = oracle.block_summaries_f32(k_u16, N, bs)
    return rne(s32.astype(np.float64)), synth.bf16_to_f32(rne(s32.astype(np.float64))).astype(
        np.float64)


def run_bf16_case(cfg, seed):
    import torch
    announce(cfg.name, "seed", seed, "B", cfg.batch, "Hq", cfg.n_q_heads, "Hkv", cfg.n_kv_heads,
             "d", cfg.head_dim, "N", cfg.seq_len, "top_k", cfg.top_k, "ratio", cfg.keep_ratio,
             "bf16 summaries")
    t = synth.gen_decode(cfg, seed)
    N, bs = cfg.seq_len, cfg.block_size
    nb = -(-N // bs)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    _, s16 = bsa.build_block_summaries(k, N, bs, want_f32=False, want_bf16=True)
    idx, scores = bsa.select_blocks(q, s16, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k,
                                    cfg.keep_ratio, want_scores=True)
    out, lse = bsa.sparse_decode_attn(q, k, v, idx, N, bs)
    out2, lse2, idx2 = bsa.sparse_decode_step(q, k, v, s16, N, bs, cfg.n_sink, cfg.n_local,
                                              cfg.top_k, cfg.keep_ratio)
    torch.cuda.synchronize()
    o_bits, o_summ = oracle_bf16_summaries(t["k"], N, bs)
    assert np.array_equal(bits(s16), o_bits), "bf16 summaries"
    o_idx, o_scores = oracle.select_blocks(t["q"], o_summ, cfg.n_kv_heads, cfg.n_sink,
                                           cfg.n_local, cfg.top_k, cfg.keep_ratio)
    g_idx = idx.cpu().numpy()
    exempt = check_index_sets(g_idx, o_idx, o_scores, nb, cfg.n_sink, cfg.n_local)
    g_sc = scores.cpu().numpy()
    cand = ~np.isnan(o_scores)
    assert np.array_equal(np.isnan(g_sc), ~cand), "scores written outside the candidates"
    bound = score_bound(t["q"], o_summ, np.zeros_like(o_summ), cfg.n_q_heads // cfg.n_kv_heads)
    assert np.all(np.abs(g_sc[cand] - o_scores[cand]) <= bound[cand]), "score error"
    o_out, o_lse, _ = oracle.sparse_decode_attn(t["q"], t["k"], t["v"], g_idx, N, bs)
    err = float(np.abs(out.cpu().numpy() - o_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - o_lse).max())
    announce("  exempt ties", exempt, "max|out err|", err, "max|lse err|", lerr)
    assert err <= OUT_ATOL and lerr <= 1e-3
    # the fused step: the same list and, bit for bit, the same outputs
    assert torch.equal(idx2, idx) and torch.equal(out2, out) and torch.equal(lse2, lse)


@pytest.mark.parametrize("g,d", [(1, 64), (4, 128), (8, 128), (16, 64)])
def test_bf16_summaries_groups_and_dims(g, d):
    cfg = synth.scaled(synth.CONFIGS["gqa32k"], name=f"bf16s_g{g}d{d}", batch=2, n_kv_heads=2,
                       n_q_heads=2 * g, head_dim=d, seq_len=64 * 150 + 37, top_k=21)
    run_bf16_case(cfg, 300 + g + d)


def test_bf16_summaries_keep_ratio_and_edges():
    base = synth.CONFIGS["gqa32k"]
    run_bf16_case(synth.scaled(base, name="bf16s_ratio", batch=2, seq_len=64 * 333 + 5,
                               top_k=-1, keep_ratio=0.15), 311)
    run_bf16_case(synth.scaled(base, name="bf16s_k0", batch=1, seq_len=64 * 40, top_k=0), 312)
    run_bf16_case(synth.scaled(base, name="bf16s_n1", batch=1, seq_len=1, top_k=3), 313)


@pytest.mark.parametrize("name", ["long128k_15", "ctx1m"])
def test_bf16_summaries_full_size(name):
    """The 128K/15 % and the 1M workloads (16,381 candidates: the top-k outside the attention
    launch) on bf16 summaries."""
    run_bf16_case(synth.CONFIGS[name], synth.DEFAULT_SEED[name])


def test_bf16_summaries_adaptive():
    """Anchor-adaptive selection on bf16 summaries: every list's count and kept set follow the
    oracle's rule on the same bf16 values (the checks of the fp32-summary adaptive tests)."""
    import torch
    cfg = synth.DecodeConfig(name="bf16s_adapt", batch=2, n_q_heads=8, n_kv_heads=4,
                             head_dim=128, seq_len=64 * 150 + 37)
    announce(cfg.name, "seed", 51, "adaptive 0.1-0.3")
    t = synth.gen_decode(cfg, 51)
    N, bs = cfg.seq_len, 64
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    _, s16 = bsa.build_block_summaries(k, N, bs, want_f32=False, want_bf16=True)
    idx, _ = bsa.select_blocks(q, s16, N, bs, 1, 2, -1, 0.1, adaptive=True, keep_ratio_max=0.3)
    out, lse = bsa.sparse_decode_attn(q, k, v, idx, N, bs)
    torch.cuda.synchronize()
    _, o_summ = oracle_bf16_summaries(t["k"], N, bs)
    o_idx, o_cnt, o_sc = oracle.select_blocks_adaptive(t["q"], o_summ, cfg.n_kv_heads, 1, 2,
                                                       0.1, 0.3, 0.0)
    g_idx = idx.cpu().numpy()
    nb = -(-N // bs)
    width, k_lo, k_hi = oracle.adaptive_bounds(nb, 1, 2, 0.1, 0.3)
    assert g_idx.shape[2] == width
    c0, c1 = 1, nb - 2
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            row = g_idx[b, h]
            cnt = int((row >= 0).sum())
            assert (row[cnt:] == -1).all() and np.all(np.diff(row[:cnt]) > 0)
            kk = cnt - 3
            assert k_lo <= kk <= k_hi
            sc = o_sc[b, h]
            anchors = np.r_[sc[:c0], sc[c1:]]
            tau = anchors.max()
            if cnt != o_cnt[b, h]:
                # only candidates within the fp32 decision's reach of tau may flip
                tol = TIE_REL * max(abs(anchors.max()), abs(anchors.min()), abs(tau), 1e-30)
                lo = int((sc[c0:c1] > tau + tol).sum())
                hi = int((sc[c0:c1] > tau - tol).sum())
                assert min(max(lo, k_lo), k_hi) <= kk <= min(max(hi, k_lo), k_hi), (b, h, cnt)
            # the kept set is the top-kk of the candidates (near-tie rule at the k-th score)
            got = set(row[:cnt].tolist()) - {0, nb - 2, nb - 1}
            want = set(oracle_topk(sc, c0, c1, kk).tolist())
            if got != want:
                kth = sc[list(want)].min()
                for j in got ^ want:
                    assert abs(sc[j] - kth) <= TIE_REL * max(abs(sc[j]), abs(kth)), (b, h, j)
    o_out, _, _ = oracle.sparse_decode_attn(t["q"], t["k"], t["v"], g_idx, N, bs)
    err = float(np.abs(out.cpu().numpy() - o_out).max())
    announce("  max|out err|", err)
    assert err <= OUT_ATOL


def test_bf16_summaries_decode_loop():
    """Per generated token on bf16 summaries with a fixed row stride: the refreshed summaries
    equal a bf16 rebuild bit for bit, and the selection and the outputs follow the oracle on
    the whole cache at every checked step."""
    import torch
    B, Hq, Hkv, d, n0, steps, cap, bs = 2, 8, 2, 128, 1000, 90, 1200, 64
    announce("bf16s_loop", "B", B, "Hq", Hq, "Hkv", Hkv, "start", n0, "steps", steps)
    cfg = synth.DecodeConfig(name="bf16s_loop", batch=B, n_q_heads=Hq, n_kv_heads=Hkv,
                             head_dim=d, seq_len=n0 + steps, top_k=9)
    t = synth.gen_decode(cfg, 321, capacity=cap)
    rng = np.random.default_rng(322)
    k_all, v_all = to_dev(t["k"]), to_dev(t["v"])
    k_cache, v_cache = torch.zeros_like(k_all), torch.zeros_like(v_all)
    k_cache[:, :, :n0] = k_all[:, :, :n0]
    v_cache[:, :, :n0] = v_all[:, :, :n0]
    S = -(-cap // bs)
    _, s16 = bsa.build_block_summaries(k_cache, n0, bs, want_f32=False, want_bf16=True,
                                       summary_stride=S)
    k_host = t["k"].copy()
    k_host[:, :, n0:] = 0
    for s in range(steps):
        N = n0 + s
        q16 = synth.bf16_round(rng.standard_normal((B, Hq, d)).astype(np.float32))
        out, lse, idx = bsa.decode_loop_step(to_dev(q16), k_all[:, :, N:N + 1].contiguous(),
                                             v_all[:, :, N:N + 1].contiguous(), k_cache, v_cache,
                                             s16, N, bs, top_k=9)
        k_host[:, :, N] = t["k"][:, :, N]
        if s % 11 and s != steps - 1:
            continue
        torch.cuda.synchronize()
        n1, nb = N + 1, -(-(N + 1) // bs)
        _, fresh = bsa.build_block_summaries(k_cache, n1, bs, want_f32=False, want_bf16=True)
        assert torch.equal(s16[:, :, :nb], fresh), f"step {s}"
        o_bits, o_summ = oracle_bf16_summaries(k_host, n1, bs)
        assert np.array_equal(bits(s16[:, :, :nb].contiguous()), o_bits), f"step {s}"
        o_idx, o_scores = oracle.select_blocks(q16, o_summ, Hkv, 1, 2, 9, 0.0)
        g_idx = idx.cpu().numpy()
        check_index_sets(g_idx, o_idx, o_scores, nb, 1, 2)
        v_host = t["v"].copy()
        v_host[:, :, n1:] = 0
        o_out, _, _ = oracle.sparse_decode_attn(q16, k_host, v_host, g_idx, n1, bs)
        assert float(np.abs(out.cpu().numpy() - o_out).max()) <= OUT_ATOL, f"step {s}"
