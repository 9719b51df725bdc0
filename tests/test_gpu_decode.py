"""GPU parity of the decode path (summaries, selection, attention) against the oracle.

Every case prints its name, seed and shapes before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import long_context_block_summary_amd as bsa
from long_context_block_summary_amd import synth
from parity_rules import (OUT_ATOL, check_index_sets, from_dev_bf16, summary_tolerance, to_dev)

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


def score_bound(q_u16, o_summ, tol_summ, g):
    """|fp32 score - exact| bound: summary error carried by |qbar| plus the fp32 dot."""
    qf = synth.bf16_to_f32(q_u16).astype(np.float64)
    B, Hq, d = qf.shape
    qbar = np.abs(qf.reshape(B, Hq // g, g, d).sum(axis=2))          # [B][Hkv][d]
    carried = np.einsum("bhc,bhjc->bhj", qbar, tol_summ)
    dot = np.einsum("bhc,bhjc->bhj", qbar, np.abs(o_summ))
    return carried + 40 * 2.0 ** -24 * dot + 1e-30


def run_decode_case(cfg, seed, capacity=None, n_splits=0):
    """Full path on the GPU vs the oracle; returns (exempted ties, max err)."""
    import torch
    announce(cfg.name, "seed", seed, "B", cfg.batch, "Hq", cfg.n_q_heads, "Hkv", cfg.n_kv_heads,
             "d", cfg.head_dim, "N", cfg.seq_len, "top_k", cfg.top_k, "splits", n_splits)
    t = synth.gen_decode(cfg, seed, capacity=capacity)
    N, bs = cfg.seq_len, cfg.block_size
    nb = -(-N // bs)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    summ, _ = bsa.build_block_summaries(k, N, bs)
    idx, scores = bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k,
                                    cfg.keep_ratio, want_scores=True)
    out, lse = bsa.sparse_decode_attn(q, k, v, idx, N, bs, n_splits=n_splits)
    torch.cuda.synchronize()
    g_summ = summ.cpu().numpy()
    g_idx = idx.cpu().numpy()
    g_out, g_lse = out.cpu().numpy(), lse.cpu().numpy()
    # summaries within the fp32 summation bound
    o_summ = oracle.block_summaries(t["k"], N, bs)
    tol = summary_tolerance(t["k"], N, bs)
    assert np.all(np.abs(g_summ - o_summ) <= tol), "summaries out of bound"
    # and bit for bit the fp32 running sum in token order divided by the count
    assert np.array_equal(g_summ, oracle.block_summaries_f32(t["k"], N, bs)), "fp32 summaries"
    # selection
    o_idx, o_scores = oracle.select_blocks(t["q"], o_summ, cfg.n_kv_heads, cfg.n_sink,
                                           cfg.n_local, cfg.top_k, cfg.keep_ratio)
    exempt = check_index_sets(g_idx, o_idx, o_scores, nb, cfg.n_sink, cfg.n_local)
    g_sc = scores.cpu().numpy()
    cand = ~np.isnan(o_scores)
    assert np.array_equal(np.isnan(g_sc), ~cand), "scores written outside the candidates"
    bound = score_bound(t["q"], o_summ, tol, cfg.n_q_heads // cfg.n_kv_heads)
    assert np.all(np.abs(g_sc[cand] - o_scores[cand]) <= bound[cand]), "score error"
    # attention against the oracle on the GPU's own index set
    o_out, o_lse, _ = oracle.sparse_decode_attn(t["q"], t["k"], t["v"], g_idx, N, bs)
    err = np.abs(g_out - o_out).max()
    lse_err = np.abs(g_lse - o_lse).max()
    announce("  exempt ties", exempt, "max|out err|", err, "max|lse err|", lse_err)
    assert err <= OUT_ATOL, err
    assert lse_err <= 1e-3, lse_err
    return exempt, err


def test_tiny_all_heads():
    cfg = synth.CONFIGS["tiny"]
    for seed in (1, 101, 102):
        run_decode_case(cfg, seed)


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_group_and_dim(g, d):
    cfg = synth.scaled(synth.CONFIGS["gqa32k"], name=f"g{g}d{d}", batch=2, n_kv_heads=2,
                       n_q_heads=2 * g, head_dim=d, seq_len=64 * 150 + 37, top_k=21)
    run_decode_case(cfg, 7 + g + d)


def test_edge_cases():
    base = synth.CONFIGS["gqa32k"]
    # k = 0: only sink + local; k beyond the candidates: every block
    run_decode_case(synth.scaled(base, name="k0", batch=1, seq_len=64 * 40, top_k=0), 31)
    run_decode_case(synth.scaled(base, name="kall", batch=1, seq_len=64 * 40, top_k=500), 32)
    # fewer blocks than sink + local, one token, a partial block
    run_decode_case(synth.scaled(base, name="nb2", batch=1, seq_len=100, top_k=5), 33)
    run_decode_case(synth.scaled(base, name="n1", batch=1, seq_len=1, top_k=5), 34)
    run_decode_case(synth.scaled(base, name="ragged", batch=3, seq_len=64 * 77 + 63, top_k=9), 35)
    # cache capacity beyond seq_len, keep ratio instead of top-k
    run_decode_case(synth.scaled(base, name="cap", batch=2, seq_len=64 * 90 + 1, top_k=-1,
                                 keep_ratio=0.15), 36, capacity=64 * 100)
    # more (batch, kv head) pairs than the plan's 256 workgroups: one split per pair
    run_decode_case(synth.scaled(base, name="manypairs", batch=40, seq_len=64 * 30 + 5, top_k=6),
                    37)


@pytest.mark.parametrize("nb", [700, 1027, 1028, 3000, 6000, 16387, 16388, 20000])
def test_topk_candidate_counts(nb):
    """Top-k over 697 .. 19997 candidates: every per-thread run length of the
    register-resident select (1, 2, 4, 8, 16 candidates per thread, with the
    1024 / 1025 and 16384 / 16385 edges) and the strided fallback beyond it.
    Random summaries compare as index sets; integer-valued ones give exact
    scores with many equal values, where the lower index must win exactly."""
    import torch
    B, Hq, Hkv, d, bs = 1, 4, 2, 128, 64
    N = nb * bs
    top_k = nb // 7
    rng = np.random.default_rng(nb)
    for kind in ("random", "integer_ties"):
        announce("topk", kind, "nb", nb, "top_k", top_k)
        if kind == "random":
            q = synth.bf16_round(rng.standard_normal((B, Hq, d)).astype(np.float32))
            summ = rng.standard_normal((B, Hkv, nb, d)).astype(np.float32)
        else:
            q = synth.bf16_round(rng.integers(-1, 2, (B, Hq, d)).astype(np.float32))
            summ = rng.integers(-2, 3, (B, Hkv, nb, d)).astype(np.float32)
        idx, scores = bsa.select_blocks(to_dev(q), torch.from_numpy(summ).cuda(), N, bs, 1, 2,
                                        top_k, want_scores=True)
        torch.cuda.synchronize()
        g_idx = idx.cpu().numpy()
        o_idx, o_scores = oracle.select_blocks(q, summ.astype(np.float64), Hkv, 1, 2, top_k)
        assert g_idx.shape == o_idx.shape
        if kind == "random":
            check_index_sets(g_idx, o_idx, o_scores, nb, 1, 2)
        else:
            assert np.array_equal(g_idx, o_idx)


def _path_summaries(kind, B, Hkv, nb, d, rng):
    """Summaries that steer the top-k down each of its paths (q is all ones, so
    every score is 2 x the row sum, an exact integer in fp32 for small rows):
    equal: every candidate score equal (zero range: radix over all keys);
    outlier: one block far above integer-valued rows (the k-th score's value
    bucket holds nearly every candidate: radix inside that bucket);
    overflow: three blocks whose fp32 scores overflow to +inf (not finite:
    radix over all keys); the oracle's fp64 scores stay finite and highest."""
    summ = rng.integers(-2, 3, (B, Hkv, nb, d)).astype(np.float32)
    if kind == "equal":
        summ[:] = 1.0
    elif kind == "outlier":
        summ[:, :, nb // 3, :] = 8192.0
    elif kind == "overflow":
        for j in (5, nb // 2, nb - 4):
            summ[:, :, j, :] = 3.0e38
    return summ


@pytest.mark.parametrize("nb", [3000, 16003])
@pytest.mark.parametrize("kind", ["equal", "outlier", "overflow"])
def test_topk_paths(kind, nb):
    """Each path of the top-k's threshold search gives the oracle's list exactly."""
    import torch
    B, Hq, Hkv, d, bs = 1, 4, 2, 128, 64
    top_k = nb // 9
    announce("topk path", kind, "nb", nb, "top_k", top_k)
    q = synth.bf16_round(np.ones((B, Hq, d), np.float32))
    summ = _path_summaries(kind, B, Hkv, nb, d, np.random.default_rng(nb))
    idx, scores = bsa.select_blocks(to_dev(q), torch.from_numpy(summ).cuda(), nb * bs, bs, 1, 2,
                                    top_k, want_scores=True)
    torch.cuda.synchronize()
    if kind == "overflow":
        assert np.isposinf(scores.cpu().numpy()[..., nb // 2]).all()
    o_idx, _ = oracle.select_blocks(q, summ.astype(np.float64), Hkv, 1, 2, top_k)
    assert np.array_equal(idx.cpu().numpy(), o_idx)


@pytest.mark.parametrize("kind", ["equal", "outlier"])
def test_topk_paths_fused_step(kind):
    """The same paths inside the attention launch (sparse_decode_step): the key
    rows of a block all equal its target summary, so the block means are it."""
    import torch
    B, Hq, Hkv, d, bs, nb = 1, 4, 2, 128, 64, 2000
    top_k = nb // 9
    announce("topk path fused", kind, "nb", nb, "top_k", top_k)
    rng = np.random.default_rng(7)
    summ = _path_summaries(kind, B, Hkv, nb, d, rng)
    k = np.repeat(summ, bs, axis=2)
    v = rng.standard_normal((B, Hkv, nb * bs, d)).astype(np.float32)
    q = synth.bf16_round(np.ones((B, Hq, d), np.float32) / 64.0)
    qd = to_dev(q)
    kd, vd = (to_dev(synth.bf16_round(a)) for a in (k, v))
    N = nb * bs
    summ_d, _ = bsa.build_block_summaries(kd, N, bs)
    idx, _ = bsa.select_blocks(qd, summ_d, N, bs, 1, 2, top_k)
    out, lse = bsa.sparse_decode_attn(qd, kd, vd, idx, N, bs)
    out2, lse2, idx2 = bsa.sparse_decode_step(qd, kd, vd, summ_d, N, bs, 1, 2, top_k, 0.0)
    torch.cuda.synchronize()
    o_idx, _ = oracle.select_blocks(q, summ.astype(np.float64), Hkv, 1, 2, top_k)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert torch.equal(idx2, idx) and torch.equal(out2, out) and torch.equal(lse2, lse)


def test_partials_then_merge_equal_the_call():
    """S4 then S5 as separate calls give sparse_decode_attn_split's result bit for bit, for
    the library's split plan and explicit split counts; the merged output is within the
    bound of the oracle."""
    import torch
    cfg = synth.scaled(synth.CONFIGS["gqa32k"], name="s4s5", batch=2, seq_len=64 * 300 + 17,
                       top_k=41)
    announce("s4s5", "B", cfg.batch, "N", cfg.seq_len)
    t = synth.gen_decode(cfg, 61)
    N, bs = cfg.seq_len, cfg.block_size
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    summ, _ = bsa.build_block_summaries(k, N, bs)
    idx, _ = bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k)
    n_keep = idx.shape[2]
    o_out, o_lse, _ = oracle.sparse_decode_attn(t["q"], t["k"], t["v"], idx.cpu().numpy(), N, bs)
    for splits in (0, 1, 3, n_keep):
        ref, ref_lse = bsa.sparse_decode_attn(q, k, v, idx, N, bs, n_splits=splits)
        ws = bsa.sparse_decode_partials(q, k, v, idx, N, bs, n_splits=splits)
        out, lse = bsa.sparse_decode_merge(ws, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads,
                                           cfg.head_dim, N, n_keep, bs, n_splits=splits,
                                           seq_stride=k.shape[2])
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), splits
        assert np.abs(out.cpu().numpy() - o_out).max() <= OUT_ATOL
        assert np.abs(lse.cpu().numpy() - o_lse).max() <= 1e-3


@pytest.mark.parametrize("name,kw", [
    ("long128k_15", {}),                                      # the headline shape, fused
    ("gqa32k", dict(batch=3, seq_len=64 * 300 + 17)),         # ragged, fused
    ("gqa32k", dict(batch=1, seq_len=64 * 40, top_k=0)),      # sink + local only
    ("gqa32k", dict(batch=1, seq_len=64 * 40, top_k=500)),    # every block
    ("gqa32k", dict(batch=1, seq_len=100, top_k=5)),          # fewer blocks than sink + local
    ("gqa32k", dict(batch=1, seq_len=64 * 3000, top_k=300)),  # 16 candidates per thread, float4 rows
    ("gqa32k", dict(batch=1, seq_len=64 * 3000 + 7, top_k=300)),  # the same, rows not float4-aligned
    ("gqa32k", dict(batch=1, seq_len=64 * 4103, top_k=400)),  # 4,100 candidates: separate launches
    ("gqa32k", dict(batch=2, n_q_heads=32, head_dim=64, seq_len=64 * 200, top_k=30)),  # d = 64
    ("gqa32k", dict(batch=2, n_kv_heads=2, n_q_heads=32, seq_len=64 * 200, top_k=30)),  # g = 16
])
def test_decode_step_equals_the_two_calls(name, kw):
    """sparse_decode_step (the selection fused into the attention launch where it fits)
    writes the list select_blocks writes and the outputs of sparse_decode_attn, bit for bit."""
    import torch
    cfg = synth.scaled(synth.CONFIGS[name], **kw)
    seed = synth.DEFAULT_SEED.get(name, 0) + 5
    announce("decode step", cfg.name, kw, "seed", seed)
    t = synth.gen_decode(cfg, seed)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    N, bs = cfg.seq_len, cfg.block_size
    summ, _ = bsa.build_block_summaries(k, N, bs)
    idx, _ = bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k,
                               cfg.keep_ratio)
    out, lse = bsa.sparse_decode_attn(q, k, v, idx, N, bs)
    for _ in range(2):  # twice: the workspace and outputs hold the previous call's values
        out2, lse2, idx2 = bsa.sparse_decode_step(q, k, v, summ, N, bs, cfg.n_sink, cfg.n_local,
                                                  cfg.top_k, cfg.keep_ratio)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx)
        assert torch.equal(out2, out)
        assert torch.equal(lse2, lse)


def test_ties_prefer_lower_index():
    import torch
    announce("ties")
    B, Hq, Hkv, d, N = 1, 8, 2, 128, 64 * 30
    k = np.zeros((B, Hkv, N, d), np.float32)
    k[..., 0] = 1.0
    k[:, :, 64 * 10:64 * 11, 0] = 3.0     # one clear winner
    v = np.random.default_rng(0).standard_normal((B, Hkv, N, d)).astype(np.float32)
    q = np.ones((B, Hq, d), np.float32)
    qd, kd, vd = (to_dev(synth.bf16_round(a)) for a in (q, k, v))
    summ, _ = bsa.build_block_summaries(kd, N, 64)
    idx, _ = bsa.select_blocks(qd, summ, N, top_k=4)
    torch.cuda.synchronize()
    expect = [0, 1, 2, 3, 10, 28, 29]
    assert idx.cpu().numpy()[0, 0].tolist() == expect
    assert idx.cpu().numpy()[0, 1].tolist() == expect


def test_split_invariance_and_determinism():
    import torch
    cfg = synth.scaled(synth.CONFIGS["long128k"], name="splits", batch=1, seq_len=64 * 512,
                       top_k=60)
    announce("split invariance", cfg)
    t = synth.gen_decode(cfg, 41)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    summ, _ = bsa.build_block_summaries(k, cfg.seq_len, 64)
    idx, _ = bsa.select_blocks(q, summ, cfg.seq_len, top_k=cfg.top_k)
    ref, ref_lse = bsa.sparse_decode_attn(q, k, v, idx, cfg.seq_len)
    again, _ = bsa.sparse_decode_attn(q, k, v, idx, cfg.seq_len)
    torch.cuda.synchronize()
    assert torch.equal(ref, again), "same plan must be bitwise reproducible"
    for s in (1, 2, 7, 16, 63):
        o, l = bsa.sparse_decode_attn(q, k, v, idx, cfg.seq_len, n_splits=s)
        torch.cuda.synchronize()
        assert (o - ref).abs().max().item() <= 1e-5, s
        assert (l - ref_lse).abs().max().item() <= 1e-5, s


def rne_bf16(x32):
    """bf16 bits of fp32 values, rounded by the oracle (nearest, ties to even)."""
    return np.vectorize(oracle.round_bf16, otypes=[np.uint16])(x32.astype(np.float64))


def test_summaries_bf16_and_compressed_block_sizes():
    import torch
    for m, N in ((4, 64 * 50 + 2), (128, 128 * 20 + 5), (64, 64 * 33)):
        announce("summaries m", m, "N", N)
        cfg = synth.scaled(synth.CONFIGS["gqa32k"], batch=1, seq_len=N)
        t = synth.gen_decode(cfg, 50 + m, capacity=N + 70)
        k = to_dev(t["k"])
        f32, b16 = bsa.build_block_summaries(k, N, m, want_f32=True, want_bf16=True)
        torch.cuda.synchronize()
        g32 = f32.cpu().numpy()
        gb = from_dev_bf16(b16)
        ref = oracle.block_summaries(t["k"], N, m)
        assert np.all(np.abs(g32 - ref) <= summary_tolerance(t["k"], N, m))
        # bit for bit: the fp32 running sum in token order / count, and its bf16 rounding
        # (nearest, ties to even)
        o32 = oracle.block_summaries_f32(t["k"], N, m)
        assert np.array_equal(g32, o32)
        assert np.array_equal(gb, rne_bf16(o32))
        # and within one bf16 step of the exact mean rounded directly
        rb = synth.bf16_to_f32(gb).astype(np.float64)
        assert np.all(np.abs(rb - ref) <= np.abs(ref) * 2.0 ** -7 + summary_tolerance(t["k"], N, m))


@pytest.mark.parametrize("name", ["gqa32k", "long128k", "long128k_15"])
def test_full_size_workloads(name):
    cfg = synth.CONFIGS[name]
    run_decode_case(cfg, synth.DEFAULT_SEED[name])


def test_full_size_1m():
    run_decode_case(synth.CONFIGS["ctx1m"], synth.DEFAULT_SEED["ctx1m"])


def test_longest_supported_cache():
    """The longest cache a decode call takes at d = 128: 2^24 tokens, so one kv head's rows
    span exactly 2^32 bytes (the kernels address them by 32-bit byte offsets from the head's
    base; one block more is BSA_UNSUPPORTED).  One kv head with 8 query heads and 262,141
    candidates (the strided top-k beyond the register kernel's 16,384), 64 of them kept:
    summaries bit for bit, scores, selection and attention against the oracle.  About a
    minute, most of it generating the 8 GiB of K and V on the host."""
    cfg = synth.scaled(synth.CONFIGS["ctx1m"], name="ctx16m", batch=1, n_q_heads=8,
                       n_kv_heads=1, seq_len=1 << 24, top_k=64)
    run_decode_case(cfg, 16)


@pytest.mark.parametrize("name", ["gqa32k", "long128k", "long128k_15", "ctx1m"])
def test_full_size_second_seed(name):
    run_decode_case(synth.CONFIGS[name], 101)


@pytest.mark.parametrize("nb,ratio", [(5, 0.7), (10, 0.35), (10, 0.45), (5, 0.9), (2048, 0.15)])
def test_keep_ratio_half_way_counts(nb, ratio):
    """Keep ratios whose product with nb sits at a rounding half-way point in double (and
    would round down from the ratio's float value): the list width and the lists equal the
    oracle's."""
    cfg = synth.scaled(synth.CONFIGS["gqa32k"], name=f"ratio{ratio}_nb{nb}", batch=2,
                       seq_len=64 * nb, top_k=-1, keep_ratio=ratio)
    run_decode_case(cfg, 200 + nb)
