"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: figures
printed on the pages, closed forms, brute force on tiny inputs, or special
cases that reduce to a library routine (numpy means, torch's
scaled_dot_product_attention in float64).  Inputs on an integer grid are used
where exact arithmetic makes the expected value unambiguous.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from long_context_block_summary_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_counts.txt")


def golden():
    vals = {}
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        key, val, kind, _cite = line.rstrip("\n").split("\t")
        vals[key] = (float(val), kind)
    return vals


def bf(x):
    """float array -> bf16 bits (values must be bf16-representable or get rounded)."""
    return synth.bf16_round(np.asarray(x, np.float32))


def f(h):
    return synth.bf16_to_f32(h).astype(np.float64)


def grid(rng, shape, lo=-4, hi=4, den=8):
    """bf16-exact values on a coarse grid (integers / den)."""
    return rng.integers(lo * den, hi * den + 1, size=shape).astype(np.float32) / den


def sdpa(q, k, v, mask=None, scale=None):
    """torch float64 SDPA; q [..., Lq, d], k/v [..., Lk, d]."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask),
        scale=scale).numpy()


# ---------------------------------------------------------------- page figures

def test_entry_counts_match_pages(orc):
    g = golden()
    for key, (val, kind) in g.items():
        if not key.startswith("entries_m"):
            continue
        m = int(key[len("entries_m"):])
        n = orc.num_blocks(1_000_000, m)
        if kind == "exact":
            assert n == int(val), key
        else:  # the page prints a rounded figure
            assert abs(n - val) <= 1, key
    # a partial block still forms an entry
    assert orc.num_blocks(1_000_000, 128) == 7813
    assert orc.num_blocks(0, 64) == 0
    assert orc.num_blocks(1, 64) == 1


def test_block_parameters_match_page_table(orc):
    g = golden()
    assert g["block_size"][0] == 64
    assert g["local_tokens"][0] == g["local_blocks"][0] * g["block_size"][0]
    # with the table's parameters the fixed part of the kept set is 3 blocks
    assert orc.num_kept(100, 1, 2, 0) == 3


def test_keep_ratio_reproduces_workload_top_k(orc):
    # the decode workloads quote both a keep ratio and a top-k; the reading
    # total = floor(r*nb + 0.5), k = total - sink - local reproduces all three
    for nb, r, k in [(512, 0.15, 74), (2048, 0.10, 202), (16384, 0.10, 1635)]:
        assert orc.num_kept(nb, 1, 2, -1, r) == k + 3
        assert orc.num_kept(nb, 1, 2, k) == k + 3
    # the 15 % variant of the 128K workload
    assert orc.num_kept(2048, 1, 2, -1, 0.15) == 307


def test_small_contexts_keep_everything(orc):
    for nb in range(0, 4):
        assert orc.num_kept(nb, 1, 2, 10) == nb
    assert orc.num_kept(4, 1, 2, 10) == 4
    assert orc.num_kept(4, 1, 2, 0) == 3


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_on_fp32_values(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 10,
                        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                                    1e-39, 3.0, 0.0])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = np.array([orc.round_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(got, ref)


def test_round_bf16_ties_to_even(orc):
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to the even mantissa (1)
    assert orc.round_bf16(1.0 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6
    assert orc.round_bf16(1.0 + 3 * 2 ** -8) == 0x3F82
    # just above a tie rounds up (the fp64 value is not first rounded to fp32)
    assert orc.round_bf16(1.0 + 2 ** -8 + 2 ** -40) == 0x3F81


# ---------------------------------------------------------------- summaries

def test_summaries_equal_numpy_mean(orc):
    rng = np.random.default_rng(1)
    B, H, N, d, bs = 2, 3, 64 * 5 + 17, 16, 64
    x = bf(rng.standard_normal((B, H, N, d)) * 3)
    s = orc.block_summaries(x, N, bs)
    xf = f(x)
    nb = -(-N // bs)
    assert s.shape == (B, H, nb, d)
    for j in range(nb):
        ref = xf[:, :, j * bs:min((j + 1) * bs, N)].mean(axis=2)
        np.testing.assert_allclose(s[:, :, j], ref, rtol=0, atol=1e-13)


def test_summaries_closed_forms(orc):
    rng = np.random.default_rng(2)
    d = 8
    row = grid(rng, (d,))
    x = np.tile(row, (1, 1, 128, 1)).astype(np.float32)
    x[0, 0, 64:] = -row
    s = orc.block_summaries(bf(x), 128, 64)
    assert np.array_equal(s[0, 0, 0], row.astype(np.float64))   # identical rows -> that row
    assert np.array_equal(s[0, 0, 1], -row.astype(np.float64))
    # block size 1 is the identity
    y = bf(rng.standard_normal((1, 2, 50, d)))
    assert np.array_equal(orc.block_summaries(y, 50, 1), f(y))
    # linearity on exact data: mean(a + b) = mean(a) + mean(b)
    a = grid(rng, (1, 1, 256, d), -2, 2)
    b = grid(rng, (1, 1, 256, d), -2, 2)
    sa, sb, sab = (orc.block_summaries(bf(z), 256, 4) for z in (a, b, a + b))
    np.testing.assert_allclose(sab, sa + sb, atol=1e-15)


def test_summaries_ignore_tokens_past_seq_len(orc):
    rng = np.random.default_rng(3)
    x = bf(rng.standard_normal((1, 1, 200, 4)))
    x2 = x.copy()
    x2[:, :, 130:] = bf(np.full((1, 1, 70, 4), 1000.0))
    assert np.array_equal(orc.block_summaries(x, 130, 64), orc.block_summaries(x2, 130, 64))


def nearest_f32(fr):
    """The fp32 value nearest to the rational fr, ties to the even significand (IEEE
    round-to-nearest-even), found by exact rational comparison of the neighbours."""
    from fractions import Fraction
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(abs(Fraction(float(x)) - fr) for x in cands)
    tied = [x for x in cands if abs(Fraction(float(x)) - fr) == best]
    return min(tied, key=lambda x: int(np.float32(x).view(np.uint32)) & 1)


def test_summaries_f32_within_the_summation_bound(orc):
    # the fp32 running sum of n values errs by at most (n - 1) u sum|x| (u = 2^-24), the
    # division adds one rounding of the quotient
    rng = np.random.default_rng(4)
    N, bs = 64 * 6 + 23, 64
    x = bf(rng.standard_normal((1, 3, N, 32)) * 5 + 2)
    s32 = orc.block_summaries_f32(x, N, bs).astype(np.float64)
    ref = orc.block_summaries(x, N, bs)
    xf = np.abs(f(x))
    for j in range(-(-N // bs)):
        n = min(bs, N - j * bs)
        bound = (n - 1) * 2.0 ** -24 * xf[:, :, j * bs:j * bs + n].sum(axis=2) / n
        bound += 2.0 ** -24 * np.abs(ref[:, :, j]) * (1 + 2.0 ** -20)
        assert np.all(np.abs(s32[:, :, j] - ref[:, :, j]) <= bound)


def test_summaries_f32_exact_on_exact_sums(orc):
    # multiples of 1/8 in [-64, 64] (bf16 keeps them multiples of 1/8): every partial sum of up
    # to 64 of them is exact in fp32,
    # so with a power-of-two count the stored mean is the exact mean
    rng = np.random.default_rng(5)
    x = grid(rng, (2, 2, 256, 16), -64, 64)
    s32 = orc.block_summaries_f32(bf(x), 256, 64)
    assert s32.dtype == np.float32
    assert np.array_equal(s32.astype(np.float64), orc.block_summaries(bf(x), 256, 64))


def test_summaries_f32_add_in_token_order(orc):
    # 2^24 then 63 ones: in fp32, 2^24 + 1 rounds back to 2^24 (ties to even), so the
    # running sum stays 2^24 and the mean is 2^18 exactly.  Ones first: 63, then
    # 63 + 2^24 = 16777279 lies halfway between 16777278 and 16777280 and rounds to the
    # even significand, 16777280; / 64 = 262145.  The exact mean, 262144.984375, is neither.
    big = 2.0 ** 24
    fwd = np.ones((1, 1, 64, 2), np.float32)
    fwd[0, 0, 0] = big
    rev = np.ones((1, 1, 64, 2), np.float32)
    rev[0, 0, 63] = big
    assert np.all(orc.block_summaries_f32(bf(fwd), 64, 64) == np.float32(262144.0))
    assert np.all(orc.block_summaries_f32(bf(rev), 64, 64) == np.float32(262145.0))
    assert np.all(orc.block_summaries(bf(fwd), 64, 64) == 262144.984375)


def test_summaries_f32_divide_once_correctly_rounded(orc):
    # partial last blocks of 3, 5, 7 and 11 tokens: the stored value is the fp32 rounding of
    # (exact integer sum) / n, not a product with a rounded reciprocal
    from fractions import Fraction
    rng = np.random.default_rng(6)
    for n in (3, 5, 7, 11):
        N = 64 + n
        x = rng.integers(-40, 41, size=(1, 1, N, 64)).astype(np.float32)
        s32 = orc.block_summaries_f32(bf(x), N, 64)
        sums = x[0, 0, 64:].astype(np.int64).sum(axis=0)
        want = np.array([nearest_f32(Fraction(int(t), n)) for t in sums], np.float32)
        assert np.array_equal(s32[0, 0, 1], want), n
    # a case where the product with the rounded reciprocal 1/3 rounds differently
    t = next(t for t in range(1, 4000)
             if np.float32(t) * np.float32(1 / 3) != nearest_f32(Fraction(t, 3)))
    x = np.zeros((1, 1, 67, 1), np.float32)
    x[0, 0, 64] = t
    assert orc.block_summaries_f32(bf(x), 67, 64)[0, 0, 1, 0] == nearest_f32(Fraction(t, 3))


# ---------------------------------------------------------------- selection

def tiny_inputs(seed=11):
    cfg = synth.CONFIGS["tiny"]
    return cfg, synth.gen_decode(cfg, seed)


def test_selection_brute_force_tiny(orc):
    cfg, t = tiny_inputs()
    s = orc.block_summaries(t["k"], cfg.seq_len, 64)
    idx, scores = orc.select_blocks(t["q"], s, cfg.n_kv_heads, 1, 2, cfg.top_k)
    nb = 16
    cand = list(range(1, nb - 2))
    for kvh in range(cfg.n_kv_heads):
        sc = scores[0, kvh]
        best = max(itertools.combinations(cand, cfg.top_k), key=lambda c: sum(sc[j] for j in c))
        assert len(list(itertools.combinations(cand, 4))) == 715
        expect = sorted([0] + list(best) + [nb - 2, nb - 1])
        assert idx[0, kvh].tolist() == expect


def test_selection_scores_from_unit_rows(orc):
    # block j's rows are all e_c, so its score is sum_h q[h][c] (a column sum of q)
    d, nb, g = 8, 12, 3
    rng = np.random.default_rng(4)
    q = grid(rng, (1, g, d))
    x = np.zeros((1, 1, nb * 64, d), np.float32)
    cols = rng.integers(0, d, nb)
    for j in range(nb):
        x[0, 0, j * 64:(j + 1) * 64, cols[j]] = 1.0
    s = orc.block_summaries(bf(x), nb * 64, 64)
    _, scores = orc.select_blocks(bf(q), s, 1, 1, 2, 3)
    for j in range(1, nb - 2):
        assert scores[0, 0, j] == pytest.approx(q[0, :, cols[j]].sum(), abs=1e-12)
    assert np.isnan(scores[0, 0, 0]) and np.isnan(scores[0, 0, nb - 1])


def test_selection_group_is_sum_of_heads(orc):
    cfg, t = tiny_inputs(12)
    s = orc.block_summaries(t["k"][:, :1], cfg.seq_len, 64)
    q = t["q"][:, :4]
    _, sg = orc.select_blocks(q, s, 1, 1, 2, 4)       # 4 query heads share kv head 0
    parts = [orc.select_blocks(q[:, h:h + 1], s, 1, 1, 2, 4)[1] for h in range(4)]
    np.testing.assert_allclose(sg, sum(parts), rtol=1e-12, atol=1e-12)


def test_selection_defining_property_and_invariants(orc):
    cfg = synth.scaled(synth.CONFIGS["gqa32k"], batch=2, seq_len=64 * 300)
    t = synth.gen_decode(cfg, 5)
    s = orc.block_summaries(t["k"], cfg.seq_len, 64)
    nb = 300
    prev = None
    for k in (0, 1, 10, 30, 31, 200, 297, 400):
        idx, sc = orc.select_blocks(t["q"], s, cfg.n_kv_heads, 1, 2, k)
        kk = min(k, nb - 3)
        assert idx.shape[-1] == kk + 3
        for b in range(2):
            for h in range(cfg.n_kv_heads):
                row = idx[b, h]
                assert np.all(np.diff(row) > 0)
                assert row[0] == 0 and row[-2] == nb - 2 and row[-1] == nb - 1
                sel = set(row.tolist()) - {0, nb - 2, nb - 1}
                uns = set(range(1, nb - 2)) - sel
                if sel and uns:
                    assert min(sc[b, h, list(sel)]) >= max(sc[b, h, list(uns)])
                if prev is not None:
                    assert set(prev[b, h].tolist()) <= set(row.tolist())  # nested in k
        prev = idx
    # scaling q by 2 (exact in bf16) keeps the selection
    q2 = bf(f(t["q"]) * 2)
    i1, s1 = orc.select_blocks(t["q"], s, cfg.n_kv_heads, 1, 2, 30)
    i2, s2 = orc.select_blocks(q2, s, cfg.n_kv_heads, 1, 2, 30)
    assert np.array_equal(i1, i2)
    np.testing.assert_allclose(s2[~np.isnan(s2)], 2 * s1[~np.isnan(s1)], rtol=1e-14)


def test_selection_sink_and_local_kept_when_lowest(orc):
    d, nb = 8, 20
    u = np.zeros(d, np.float32)
    u[0] = 1
    x = np.zeros((1, 1, nb * 64, d), np.float32)
    for j in range(nb):
        x[0, 0, j * 64:(j + 1) * 64, 0] = 1.0 + j % 5
    x[0, 0, :64, 0] = -50          # sink block scores lowest
    x[0, 0, -128:, 0] = -50        # local blocks score lowest
    x[0, 0, 7 * 64:8 * 64, 0] = 40  # needle
    q = np.tile(u, (1, 1, 1))
    s = orc.block_summaries(bf(x), nb * 64, 64)
    idx, _ = orc.select_blocks(bf(q), s, 1, 1, 2, 1)
    assert idx[0, 0].tolist() == [0, 7, nb - 2, nb - 1]


def test_selection_ties_prefer_lower_index(orc):
    d, nb = 4, 12
    x = np.zeros((1, 1, nb * 64, d), np.float32)
    x[..., 0] = 1.0            # every block has the same summary
    q = np.ones((1, 1, d), np.float32)
    s = orc.block_summaries(bf(x), nb * 64, 64)
    idx, _ = orc.select_blocks(bf(q), s, 1, 1, 2, 3)
    assert idx[0, 0].tolist() == [0, 1, 2, 3, 10, 11]


# ---------------------------------------------------------------- decode attention

def gather_tokens(idx_row, bs, N):
    return np.concatenate([np.arange(j * bs, min((j + 1) * bs, N)) for j in idx_row])


def test_all_blocks_equal_dense_sdpa(orc):
    cfg, t = tiny_inputs(13)
    s = orc.block_summaries(t["k"], cfg.seq_len, 64)
    idx, _ = orc.select_blocks(t["q"], s, cfg.n_kv_heads, 1, 2, 13)   # k covers every block
    assert idx.shape[-1] == 16
    out, lse, w = orc.sparse_decode_attn(t["q"], t["k"], t["v"], idx, cfg.seq_len,
                                         want_weights=True)
    q, k, v = f(t["q"]), f(t["k"]), f(t["v"])
    ref = sdpa(q[0][:, None, :], k[0], v[0])[:, 0, :]
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(w.sum(-1), 1.0, atol=1e-12)


def test_gqa_partial_selection_equals_sdpa_over_gathered(orc):
    cfg = synth.scaled(synth.CONFIGS["gqa32k"], batch=2, seq_len=64 * 40 + 23, head_dim=64)
    t = synth.gen_decode(cfg, 6)
    nb = 41
    s = orc.block_summaries(t["k"], cfg.seq_len, 64)
    idx, _ = orc.select_blocks(t["q"], s, cfg.n_kv_heads, 1, 2, 6)
    out, lse, _ = orc.sparse_decode_attn(t["q"], t["k"], t["v"], idx, cfg.seq_len)
    q, k, v = f(t["q"]), f(t["k"]), f(t["v"])
    g = cfg.n_q_heads // cfg.n_kv_heads
    assert idx[0, 0, -1] == nb - 1   # the partial last block is local
    for b in range(2):
        for h in range(cfg.n_q_heads):
            toks = gather_tokens(idx[b, h // g], 64, cfg.seq_len)
            ref = sdpa(q[b, h][None], k[b, h // g, toks], v[b, h // g, toks])[0]
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


def test_weights_equal_sdpa_with_identity_values(orc):
    # with V_t = e_t the attention output is the weight vector itself
    rng = np.random.default_rng(7)
    d, N = 64, 64
    q = bf(rng.standard_normal((1, 1, d)))
    k = bf(rng.standard_normal((1, 1, N, d)) * 2)
    v = bf(np.eye(N, d, dtype=np.float32)[None, None])
    idx = np.zeros((1, 1, 1), np.int32)
    out, lse, w = orc.sparse_decode_attn(q, k, v, idx, N, want_weights=True)
    ref = sdpa(f(q)[0], f(k)[0, 0], np.eye(N))[0]
    np.testing.assert_allclose(w[0, 0], ref, atol=1e-14)
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-14)


def test_decode_closed_forms(orc):
    rng = np.random.default_rng(8)
    d, N = 16, 256
    v = bf(rng.standard_normal((1, 1, N, d)))
    q = bf(rng.standard_normal((1, 2, d)))
    idx = np.array([[[0, 2, 3]]], np.int32)
    # zero keys: uniform weights -> mean of the kept values; lse = log(#tokens)
    out, lse, _ = orc.sparse_decode_attn(q, bf(np.zeros((1, 1, N, d))), v, idx, N)
    toks = gather_tokens(idx[0, 0], 64, N)
    np.testing.assert_allclose(out[0, 0], f(v)[0, 0, toks].mean(0), atol=1e-14)
    assert lse[0, 1] == pytest.approx(math.log(len(toks)), abs=1e-14)
    # one dominant logit -> that token's value
    k = np.zeros((1, 1, N, d), np.float32)
    k[0, 0, 150] = 64 * f(q)[0, 0] / max(1e-3, np.abs(f(q)[0, 0]).max())
    out, _, _ = orc.sparse_decode_attn(q[:, :1], bf(k), v, idx, N)
    np.testing.assert_allclose(out[0, 0], f(v)[0, 0, 150], atol=1e-9)


def test_decode_linear_in_v_and_scale_default(orc):
    rng = np.random.default_rng(9)
    d, N = 32, 192
    q = bf(rng.standard_normal((1, 2, d)))
    k = bf(rng.standard_normal((1, 1, N, d)))
    v1, v2 = grid(rng, (1, 1, N, d), -2, 2), grid(rng, (1, 1, N, d), -2, 2)
    idx = np.array([[[0, 2]]], np.int32)
    o1, _, _ = orc.sparse_decode_attn(q, k, bf(v1), idx, N)
    o2, _, _ = orc.sparse_decode_attn(q, k, bf(v2), idx, N)
    o12, _, _ = orc.sparse_decode_attn(q, k, bf(v1 + v2), idx, N)
    np.testing.assert_allclose(o12, o1 + o2, atol=1e-13)
    oa, la, _ = orc.sparse_decode_attn(q, k, bf(v1), idx, N, scale=0.0)
    ob, lb, _ = orc.sparse_decode_attn(q, k, bf(v1), idx, N, scale=1 / math.sqrt(d))
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_lse_merges_disjoint_sets(orc):
    # softmax over A u B from the parts: o = (e^lA oA + e^lB oB) / (e^lA + e^lB)
    rng = np.random.default_rng(10)
    d, N = 32, 64 * 6
    q = bf(rng.standard_normal((1, 2, d)))
    k = bf(rng.standard_normal((1, 1, N, d)) * 2)
    v = bf(rng.standard_normal((1, 1, N, d)))
    oa, la, _ = orc.sparse_decode_attn(q, k, v, np.array([[[0, 3]]], np.int32), N)
    ob, lb, _ = orc.sparse_decode_attn(q, k, v, np.array([[[1, 5]]], np.int32), N)
    oab, lab, _ = orc.sparse_decode_attn(q, k, v, np.array([[[0, 1, 3, 5]]], np.int32), N)
    wa, wb = np.exp(la - lab)[..., None], np.exp(lb - lab)[..., None]
    np.testing.assert_allclose(wa + wb, 1.0, atol=1e-12)
    np.testing.assert_allclose(oab, wa * oa + wb * ob, atol=1e-12)


def test_decode_rejects_bad_index_lists(orc):
    q = np.zeros((1, 1, 8), np.uint16)
    k = np.zeros((1, 1, 128, 8), np.uint16)
    for bad in ([[[1, 1]]], [[[1, 0]]], [[[0, 2]]], [[[-1, 0]]]):
        with pytest.raises(ValueError):
            orc.sparse_decode_attn(q, k, k, np.array(bad, np.int32), 128)


# ---------------------------------------------------------------- prefill

def prefill_case(seed, P=256, C=40, Hq=4, Hkv=2, d=16, exact=True):
    rng = np.random.default_rng(seed)
    n = P + C
    if exact:
        k = grid(rng, (1, Hkv, n, d), -2, 2, 4)
        v = grid(rng, (1, Hkv, n, d), -2, 2, 4)
    else:
        k = rng.standard_normal((1, Hkv, n, d)).astype(np.float32)
        v = rng.standard_normal((1, Hkv, n, d)).astype(np.float32)
    q = rng.standard_normal((1, C, Hq, d)).astype(np.float32)
    return bf(q), bf(k), bf(v)


def test_prefill_branch_b_m1_is_dense_attention(orc):
    q, k, v = prefill_case(20)
    P = 256
    r = orc.sparse_prefill_attn(q, k, v, P, m_sparse=4, top_k=8, m_dense=1, window=4,
                                q_tile=16, want_branches=True)
    qf, kf, vf = f(q), f(k), f(v)
    for h in range(4):
        ref = sdpa(qf[0, :, h], kf[0, h // 2, :P], vf[0, h // 2, :P])
        np.testing.assert_allclose(r["branches"][1, 0, :, h], ref, atol=1e-12)


def test_prefill_branch_a_all_entries_is_dense_over_pooled(orc):
    q, k, v = prefill_case(21)
    P, m = 256, 2
    r = orc.sparse_prefill_attn(q, k, v, P, m_sparse=m, top_k=10 ** 6, m_dense=64, window=4,
                                q_tile=16, want_branches=True, want_sel=True)
    assert r["sel"].shape[-1] == P // m
    qf, kf, vf = f(q), f(k), f(v)
    # grid data: the pooled means are exact in bf16, so numpy's mean is the operand
    kp = kf[0, :, :P].reshape(2, P // m, m, -1).mean(2)
    vp = vf[0, :, :P].reshape(2, P // m, m, -1).mean(2)
    assert np.array_equal(f(bf(kp)), kp) and np.array_equal(f(bf(vp)), vp)
    for h in range(4):
        ref = sdpa(qf[0, :, h], kp[h // 2], vp[h // 2])
        np.testing.assert_allclose(r["branches"][0, 0, :, h], ref, atol=1e-12)


def test_prefill_compressed_operands_are_bf16_rounded_means(orc):
    # "CSA + HCA 混合注意力机制" §4.1 / §5.1: an entry is the mean of m consecutive rows;
    # the attention copies of the entries are a bf16 cache (round to nearest even of the
    # mean).  Values n/64 with |n| <= 255 are bf16-exact, and the mean of 4 of them,
    # (sum of n)/256, has up to 10 significant bits: exact in fp32 but mostly not in bf16,
    # so the rounding (ties included) decides both branches' operands.  torch's fp32 ->
    # bf16 conversion rounds them independently of the oracle.
    rng = np.random.default_rng(28)
    P, C, Hq, Hkv, d, m = 256, 40, 4, 2, 16, 4
    k = rng.integers(-255, 256, (1, Hkv, P + C, d)).astype(np.float32) / 64
    v = rng.integers(-255, 256, (1, Hkv, P + C, d)).astype(np.float32) / 64
    q = rng.standard_normal((1, C, Hq, d)).astype(np.float32)
    qb, kb, vb = bf(q), bf(k), bf(v)
    assert np.array_equal(f(kb), k) and np.array_equal(f(vb), v)
    kp = k[0, :, :P].astype(np.float64).reshape(Hkv, P // m, m, d).mean(2)
    vp = v[0, :, :P].astype(np.float64).reshape(Hkv, P // m, m, d).mean(2)
    assert np.array_equal(kp.astype(np.float32), kp) and np.array_equal(vp.astype(np.float32), vp)

    def rne(a):
        return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).double().numpy()

    kr, vr = rne(kp), rne(vp)
    assert (kr != kp).mean() > 0.15 and (vr != vp).mean() > 0.15
    # some means lie exactly halfway between two bf16 values (the 16 fp32 bits that bf16
    # drops are 0x8000)
    half = lambda a: (a.astype(np.float32).view(np.uint32) & 0xFFFF) == 0x8000
    assert half(kp).sum() > 10 and half(vp).sum() > 10
    # branch A over every m=4 entry and branch B with m_dense = 4 attend the same stream
    r = orc.sparse_prefill_attn(qb, kb, vb, P, m_sparse=m, top_k=10 ** 6, m_dense=m, window=4,
                                q_tile=16, want_branches=True)
    qf = f(qb)
    for h in range(Hq):
        ref = sdpa(qf[0, :, h], kr[h // 2], vr[h // 2])
        np.testing.assert_allclose(r["branches"][0, 0, :, h], ref, atol=1e-12)
        np.testing.assert_allclose(r["branches"][1, 0, :, h], ref, atol=1e-12)
        # the unrounded means give a visibly different result
        assert np.abs(sdpa(qf[0, :, h], kp[h // 2], vp[h // 2]) - ref).max() > 1e-5


def test_prefill_branch_c_window(orc):
    q, k, v = prefill_case(22, exact=False)
    P, C = 256, 40
    big = orc.sparse_prefill_attn(q, k, v, P, top_k=8, window=P + C, q_tile=16,
                                  want_branches=True)
    qf, kf, vf = f(q), f(k), f(v)
    pos = P + np.arange(C)
    mask = np.arange(P + C)[None, :] <= pos[:, None]          # causal
    for h in range(4):
        ref = sdpa(qf[0, :, h], kf[0, h // 2], vf[0, h // 2], mask=mask)
        np.testing.assert_allclose(big["branches"][2, 0, :, h], ref, atol=1e-12)
    one = orc.sparse_prefill_attn(q, k, v, P, top_k=8, window=1, q_tile=16, want_branches=True)
    for h in range(4):
        np.testing.assert_array_equal(one["branches"][2, 0, :, h], vf[0, h // 2, P:P + C])
    # window 128 covers [p-127, p]
    w = orc.sparse_prefill_attn(q, k, v, P, top_k=8, window=128, q_tile=16, want_branches=True)
    mask = (np.arange(P + C)[None, :] <= pos[:, None]) & (np.arange(P + C)[None, :] > pos[:, None] - 128)
    ref = sdpa(qf[0, :, 3], kf[0, 1], vf[0, 1], mask=mask)
    np.testing.assert_allclose(w["branches"][2, 0, :, 3], ref, atol=1e-12)


def test_prefill_average_and_rows(orc):
    q, k, v = prefill_case(23, exact=False)
    P = 256
    full = orc.sparse_prefill_attn(q, k, v, P, top_k=8, m_dense=32, window=16, q_tile=16,
                                   want_branches=True, want_sel=True)
    br = full["branches"]
    np.testing.assert_allclose(full["out"], (br[0] + br[1] + br[2]) / 3, atol=1e-15)
    rows = np.array([39, 0, 17, 16])
    part = orc.sparse_prefill_attn(q, k, v, P, top_k=8, m_dense=32, window=16, q_tile=16,
                                   rows=rows)
    np.testing.assert_array_equal(part["out"][0], full["out"][0, rows])
    again = orc.sparse_prefill_attn(q, k, v, P, top_k=8, m_dense=32, window=16, q_tile=16,
                                    sel_in=full["sel"])
    np.testing.assert_array_equal(again["out"], full["out"])


def test_prefill_tile_selection(orc):
    P, C, d, m = 256, 48, 8, 4
    E = P // m
    k = np.zeros((1, 1, P + C, d), np.float32)
    k[0, 0, :P, 1] = np.arange(P) % 7 * 0.25        # mild structure everywhere
    k[0, 0, 20 * m:21 * m, 0] = 8.0                  # entry 20 points along +e0
    k[0, 0, 33 * m:34 * m, 0] = -8.0                 # entry 33 points along -e0
    q = np.zeros((1, C, 1, d), np.float32)
    q[0, :16, 0, 0] = 1.0                            # tile 0 looks along +e0
    q[0, 16:32, 0, 0] = -1.0                         # tile 1 looks along -e0
    q[0, 32:, 0, 1] = 1.0                            # tile 2 looks along e1
    r = orc.sparse_prefill_attn(bf(q), bf(k), bf(k), P, m_sparse=m, top_k=1, q_tile=16,
                                want_sel=True, want_sel_scores=True)
    assert r["sel"][0, :, 0, 0].tolist()[:2] == [20, 33]
    ss = r["sel_scores"][0, 2, 0]
    assert r["sel"][0, 2, 0, 0] == int(np.argmax(ss))            # first of the maxima
    r8 = orc.sparse_prefill_attn(bf(q), bf(k), bf(k), P, m_sparse=m, top_k=8, q_tile=16,
                                 want_sel=True, want_sel_scores=True)
    for t in range(3):
        sel = r8["sel"][0, t, 0]
        sc = r8["sel_scores"][0, t, 0]
        assert np.all(np.diff(sel) > 0)
        uns = np.setdiff1d(np.arange(E), sel)
        assert sc[sel].min() >= sc[uns].max()
        # ties resolve to the lower index
        tied = uns[sc[uns] == sc[sel].min()]
        assert np.all(tied > sel[sc[sel] == sc[sel].min()].max())


def _indexer_case(tokens0, tokens1, d=8):
    """Two m = 4 entries whose first dim holds the given tokens (others zero) and one
    query along +e0: each entry's score is its key's first component."""
    P, m = 8, 4
    k = np.zeros((1, 1, P + 1, d), np.float32)
    k[0, 0, :m, 0] = tokens0
    k[0, 0, m:P, 0] = tokens1
    q = np.zeros((1, 1, 1, d), np.float32)
    q[0, 0, 0, 0] = 1.0
    assert np.array_equal(f(bf(k)), k)  # every token is a bf16 value
    return bf(q), bf(k), P, m


def test_prefill_indexer_scores_bf16_keys(orc):
    # "CSA + HCA 混合注意力机制" §4.2: the indexer scores the compressed entries at low
    # precision, its recall measured against a BF16 indexer.  Entry 1's mean
    # 1 + 2^-9 rounds to the bf16 value 1 (the half ulp is 2^-8): with bf16 keys the
    # two entries tie and the lower index wins; with the exact means entry 1 wins.
    q, k, P, m = _indexer_case([1.0] * 4, [1.0, 1.0, 1.0, 1.0 + 2.0 ** -7])
    kw = dict(m_sparse=m, top_k=1, m_dense=m, window=1, want_sel=True, want_sel_scores=True)
    r = orc.sparse_prefill_attn(q, k, k, P, indexer=0, **kw)
    assert r["sel"][0, 0, 0].tolist() == [0]
    assert r["sel_scores"][0, 0, 0].tolist() == [1.0, 1.0]
    r = orc.sparse_prefill_attn(q, k, k, P, indexer=1, **kw)
    assert r["sel"][0, 0, 0].tolist() == [1]
    assert r["sel_scores"][0, 0, 0].tolist() == [1.0, 1.0 + 2.0 ** -9]


def test_prefill_indexer_keys_round_the_fp32_token_order_mean(orc):
    # the bf16 keys are the stream as stored: the fp32 running sum in token order,
    # divided by the count, then rounded to bf16.  Entry 0's tokens 2^20, 1 + 2^-7,
    # -2^20, 0 sum in fp32 to 1 (2^20 + 1 + 2^-7 rounds to 2^20 + 1: its ulp is 2^-3),
    # so its key is 0.25, below entry 1's 0.25 + 2^-9; rounding the exact mean
    # (0.25 + 2^-9) instead would tie the two and pick entry 0.
    q, k, P, m = _indexer_case([2.0 ** 20, 1.0 + 2.0 ** -7, -(2.0 ** 20), 0.0],
                               [0.25 + 2.0 ** -9] * 4)
    kw = dict(m_sparse=m, top_k=1, m_dense=m, window=1, want_sel=True, want_sel_scores=True)
    r = orc.sparse_prefill_attn(q, k, k, P, indexer=0, **kw)
    assert r["sel_scores"][0, 0, 0].tolist() == [0.25, 0.25 + 2.0 ** -9]
    assert r["sel"][0, 0, 0].tolist() == [1]
    r = orc.sparse_prefill_attn(q, k, k, P, indexer=1, **kw)
    assert r["sel_scores"][0, 0, 0].tolist() == [0.25 + 2.0 ** -9] * 2
    assert r["sel"][0, 0, 0].tolist() == [0]


def test_prefill_tile_scores_from_unit_entries(orc):
    # entry j's rows are all e_{c_j}: its score for a tile is the sum of q[., ., c_j]
    # over the tile's queries and the kv head's query heads (ragged last tile too)
    P, C, d, m, Hq, Hkv, qt = 128, 40, 8, 4, 4, 2, 16
    E = P // m
    rng = np.random.default_rng(24)
    cols = rng.integers(0, d, E)
    k = np.zeros((1, Hkv, P + C, d), np.float32)
    for j in range(E):
        k[0, :, j * m:(j + 1) * m, cols[j]] = 1.0
    q = grid(rng, (1, C, Hq, d))
    r = orc.sparse_prefill_attn(bf(q), bf(k), bf(k), P, m_sparse=m, top_k=3, q_tile=qt,
                                want_sel_scores=True)
    ss = r["sel_scores"][0]
    for t in range(3):
        for kvh in range(Hkv):
            qs = q[0, t * qt:min((t + 1) * qt, C), kvh * 2:kvh * 2 + 2].sum(axis=(0, 1))
            np.testing.assert_allclose(ss[t, kvh], qs[cols], atol=1e-12)


# ------------------------------------------- branch combination and sink logits
# "CSA + HCA 混合注意力机制" §4.3 attends the compressed entries, the window and the
# tail in one softmax; §5.4 adds a learnable sink logit (no value) to the softmax.

def _lse(x, axis=0):
    m = np.max(x, axis=axis, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(axis=axis, keepdims=True))).squeeze(axis)


def test_prefill_concat_is_lse_weighted_branches(orc):
    # one softmax over the concatenated logits = sum_X e^(lse_X - L) o_X,
    # L = log sum_X e^(lse_X); the concat path computes its logits itself
    q, k, v = prefill_case(25, exact=False)
    P = 256
    kw = dict(top_k=8, m_dense=32, window=20, q_tile=16, want_branches=True)
    r = orc.sparse_prefill_attn(q, k, v, P, combine=1, **kw)
    lse3, br = r["lse3"], r["branches"]
    L = _lse(lse3, axis=0)
    ref = (np.exp(lse3 - L)[..., None] * br).sum(axis=0)
    np.testing.assert_allclose(r["out"], ref, atol=1e-12)
    # the branches themselves do not depend on the combination
    r0 = orc.sparse_prefill_attn(q, k, v, P, combine=0, **kw)
    np.testing.assert_array_equal(r0["branches"], br)
    np.testing.assert_array_equal(r0["lse3"], lse3)


def test_prefill_sink_closed_forms(orc):
    q, k, v = prefill_case(26, exact=False)
    P, Hq = 256, 4
    kw = dict(top_k=8, m_dense=32, window=20, q_tile=16, want_branches=True)
    z = np.array([-1.5, 0.0, 2.0, 7.0])
    for combine in (0, 1):
        base = orc.sparse_prefill_attn(q, k, v, P, combine=combine, **kw)
        # a sink logit far below every logit changes nothing
        far = orc.sparse_prefill_attn(q, k, v, P, combine=combine,
                                      sink_logits=np.full(Hq, -1e300), **kw)
        np.testing.assert_array_equal(far["out"], base["out"])
        # a sink logit far above every logit takes all the mass
        big = orc.sparse_prefill_attn(q, k, v, P, combine=combine,
                                      sink_logits=np.full(Hq, 1e3), **kw)
        assert np.abs(big["out"]).max() < 1e-300
        r = orc.sparse_prefill_attn(q, k, v, P, combine=combine, sink_logits=z, **kw)
        lse3, br = base["lse3"], base["branches"]
        if combine == 0:
            # each branch keeps e^lse / (e^lse + e^z) of its mass
            keep = 1.0 / (1.0 + np.exp(z[None, None, None, :] - lse3))
            ref = (keep[..., None] * br).sum(axis=0) / 3.0
        else:
            L = _lse(lse3, axis=0)
            ref = base["out"] / (1.0 + np.exp(z[None, None, :] - L))[..., None]
        np.testing.assert_allclose(r["out"], ref, atol=1e-12)
    # a sink logit equal to a branch's lse halves that branch (single branch view)
    one = orc.sparse_prefill_attn(q, k, v, P, combine=0, **kw)
    h_lse = one["lse3"][0, 0, 5, :]  # branch A, query 5, every head
    rows = np.array([5], np.int32)
    rr = orc.sparse_prefill_attn(q, k, v, P, combine=0, rows=rows, sink_logits=h_lse, **kw)
    keep = 1.0 / (1.0 + np.exp(h_lse[None, :] - one["lse3"][:, 0, 5, :]))
    assert np.allclose(keep[0], 0.5, atol=1e-15)
    ref = (keep[..., None] * one["branches"][:, 0, 5]).sum(axis=0) / 3.0
    np.testing.assert_allclose(rr["out"][0, 0], ref, atol=1e-12)


def test_prefill_combine_rejects_unknown_mode(orc):
    q, k, v = prefill_case(27)
    with pytest.raises(ValueError):
        orc.sparse_prefill_attn(q, k, v, 256, top_k=8, combine=2)


# ------------------------------------------------- anchor-adaptive selection
# hotdry.top post: the sink and local blocks are anchors; blocks whose importance
# exceeds the anchor point are kept, within a 10-20 % keep range.

def _adaptive_case(cand_scores, anchor_scores, d=4):
    """Summaries whose column 0 carries the scores (q = e_0, one head): block 0 and the
    last two blocks are the anchors."""
    nb = len(cand_scores) + 3
    summ = np.zeros((1, 1, nb, d))
    summ[0, 0, 0, 0] = anchor_scores[0]
    summ[0, 0, 1:nb - 2, 0] = cand_scores
    summ[0, 0, nb - 2:, 0] = anchor_scores[1:]
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    return bf(q), summ, nb


def test_adaptive_bounds_reproduce_the_keep_range(orc):
    # 10 % and 20 % of 2048 blocks with sink 1 + local 2: k in [202, 407]
    assert orc.adaptive_bounds(2048, 1, 2, 0.1, 0.2) == (410, 202, 407)
    assert orc.adaptive_bounds(512, 1, 2, 0.15, 0.15) == (77, 74, 74)
    # tiny contexts keep everything; an inverted range is rejected
    assert orc.adaptive_bounds(3, 1, 2, 0.1, 0.2) == (3, 0, 0)
    with pytest.raises(ValueError):
        orc.adaptive_bounds(100, 1, 2, 0.3, 0.2)


def test_adaptive_count_above_the_anchor_threshold(orc):
    rng = np.random.default_rng(31)
    cand = rng.permutation(np.arange(37, dtype=np.float64)) * 0.25  # 0 .. 9, distinct
    anchors = [2.0, 1.0, 3.0]                                       # a_max 3, a_min 1
    q, summ, nb = _adaptive_case(cand, anchors)
    width, k_lo, k_hi = orc.adaptive_bounds(nb, 1, 2, 0.1, 0.5)
    assert (k_lo, k_hi) == (1, 17)
    for margin, tau in ((0.0, 3.0), (1.0, 5.0), (0.5, 4.0), (-0.25, 2.5), (3.0, 9.0)):
        idx, cnt, sc = orc.select_blocks_adaptive(q, summ, 1, 1, 2, 0.1, 0.5, margin)
        above = int((cand > tau).sum())              # strictly above: a score equal to tau is out
        k = min(max(above, k_lo), k_hi)
        assert cnt[0, 0] == 3 + k
        expect = sorted([0, nb - 2, nb - 1] + [1 + j for j in np.argsort(-cand, kind="stable")[:k]])
        assert idx[0, 0, :3 + k].tolist() == expect
        assert (idx[0, 0, 3 + k:] == -1).all() and idx.shape[2] == width
        np.testing.assert_allclose(sc[0, 0, 1:nb - 2], cand, atol=0)


def test_adaptive_all_equal_scores_keep_the_minimum(orc):
    q, summ, nb = _adaptive_case(np.full(60, 1.5), [1.5, 1.5, 1.5])
    _, k_lo, _ = orc.adaptive_bounds(nb, 1, 2, 0.1, 0.2)
    idx, cnt, _ = orc.select_blocks_adaptive(q, summ, 1, 1, 2, 0.1, 0.2, 0.0)
    assert cnt[0, 0] == 3 + k_lo
    # equal scores: the lowest candidate indices
    assert idx[0, 0, :3 + k_lo].tolist() == [0] + list(range(1, 1 + k_lo)) + [nb - 2, nb - 1]


def test_adaptive_anchors_include_the_local_blocks(orc):
    # raising a local block's score raises the threshold: fewer blocks kept, never more
    cand = np.linspace(0.0, 10.0, 50)
    prev = None
    for local in (0.0, 4.0, 7.0, 9.5):
        q, summ, nb = _adaptive_case(cand, [1.0, local, 0.5])
        _, cnt, _ = orc.select_blocks_adaptive(q, summ, 1, 1, 2, 0.0, 1.0, 0.0)
        assert cnt[0, 0] == 3 + int((cand > max(1.0, local)).sum())
        assert prev is None or cnt[0, 0] <= prev
        prev = cnt[0, 0]


def test_padded_lists_attend_like_truncated_ones(orc):
    rng = np.random.default_rng(33)
    q = bf(rng.standard_normal((1, 2, 16)).astype(np.float32))
    k = bf(rng.standard_normal((1, 2, 64 * 9, 16)).astype(np.float32))
    v = bf(rng.standard_normal((1, 2, 64 * 9, 16)).astype(np.float32))
    full = np.array([[[0, 3, 4, 8, -1, -1], [1, 2, 5, 6, 7, 8]]], np.int32)
    o_pad, l_pad, _ = orc.sparse_decode_attn(q, k, v, full, 64 * 9 - 5)
    o_a, l_a, _ = orc.sparse_decode_attn(q[:, :1], k[:, :1], v[:, :1], full[:, :1, :4], 64 * 9 - 5)
    np.testing.assert_array_equal(o_pad[:, :1], o_a)
    np.testing.assert_array_equal(l_pad[:, :1], l_a)
    for bad in ([[[-1, -1]]], [[[2, -1, 3]]], [[[0, -1, -1, 1]]]):
        with pytest.raises(ValueError):
            orc.sparse_decode_attn(q[:, :1], k[:, :1], v[:, :1], np.array(bad, np.int32), 128)


# ------------------------------------------------------------- FP8 KV cache
# aicoding.csdn.net page, 二.2 (3): the KV cache stored in FP8.  The format is not
# fixed there: OCP E4M3 with one scale per (pair, block); torch's float8_e4m3fn is
# an independent implementation of the same format.

def test_e4m3_values_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([orc.e4m3_value(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e4m3_encoding_matches_torch_incl_ties(orc):
    rng = np.random.default_rng(41)
    vals = (rng.uniform(-448, 448, 3000) * np.exp2(rng.integers(-12, 1, 3000))).astype(np.float32)
    # every midpoint between adjacent finite codes (a tie: even code wins)
    fin = np.array(sorted({orc.e4m3_value(c) for c in range(0, 127)}))
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([vals, mids, -mids, [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(v) for v in vals], np.uint8)
    np.testing.assert_array_equal(got, ref)
    # beyond the largest finite value the oracle saturates (torch would give NaN)
    assert orc.e4m3_encode(449.0) == 0x7E and orc.e4m3_encode(-1e9) == 0xFE


def test_quantize_fp8_closed_forms(orc):
    rng = np.random.default_rng(42)
    fin = np.array(sorted({orc.e4m3_value(c) for c in range(0, 127)}))
    d, bs = 16, 64
    # block 0: E4M3 values whose amax is 448 -> scale 1, codes exact;
    # block 1: the same times 2^-5 -> scale 2^-5, same codes; block 2: zeros;
    # block 3 (partial, 10 tokens): general values
    b0 = rng.choice(np.concatenate([fin, -fin]), (bs, d)).astype(np.float32)
    b0[3, 5] = 448.0
    x = np.zeros((1, 1, 4 * bs, d), np.float32)
    x[0, 0, :bs] = b0
    x[0, 0, bs:2 * bs] = b0 * 2.0 ** -5
    x[0, 0, 3 * bs:3 * bs + 10] = rng.standard_normal((10, d))
    N = 3 * bs + 10
    codes, sc = orc.quantize_fp8(bf(x), N, bs)
    assert sc[0, 0, 0] == 1.0 and sc[0, 0, 1] == 2.0 ** -5 and sc[0, 0, 2] == 0.0
    np.testing.assert_array_equal(codes[0, 0, :bs], codes[0, 0, bs:2 * bs])
    val = np.vectorize(orc.e4m3_value)
    np.testing.assert_array_equal(val(codes[0, 0, :bs]), b0)
    assert not codes[0, 0, 2 * bs:3 * bs].any() and not codes[0, 0, N:].any()
    # the general block: within half a code spacing, and its amax maps to 448
    xb = f(bf(x))[0, 0, 3 * bs:N]
    deq = sc[0, 0, 3] * val(codes[0, 0, 3 * bs:N])
    assert np.all(np.abs(deq - xb) <= np.maximum(2.0 ** -4 * np.abs(xb), sc[0, 0, 3] * 2.0 ** -10)
                  * (1 + 1e-6))
    assert np.abs(val(codes[0, 0, 3 * bs:N])).max() == 448.0


def test_fp8_attention_equals_bf16_on_representable_cache(orc):
    # a cache of E4M3 values with 448 in every block quantizes exactly (scale 1):
    # attention over it must equal the bf16 path on the same values
    rng = np.random.default_rng(43)
    fin = np.array(sorted({orc.e4m3_value(c) for c in range(0, 127)}))
    pool = np.concatenate([fin[(fin > 0.05) & (fin < 4)], -fin[(fin > 0.05) & (fin < 4)]])
    B, Hq, Hkv, d, N = 1, 4, 2, 16, 64 * 6 - 7
    k = rng.choice(pool, (B, Hkv, N, d)).astype(np.float32)
    v = rng.choice(pool, (B, Hkv, N, d)).astype(np.float32)
    for j in range(6):
        k[:, :, j * 64, 0] = 448.0
        v[:, :, j * 64, 1] = 448.0
    q = bf(rng.standard_normal((B, Hq, d)).astype(np.float32) * 0.01)
    k16, v16 = bf(k), bf(v)
    k8, ks = orc.quantize_fp8(k16, N)
    v8, vs = orc.quantize_fp8(v16, N)
    assert (ks == 1.0).all() and (vs == 1.0).all()
    idx = np.array([[[0, 2, 3, 5], [1, 2, 4, 5]]], np.int32)
    o8, l8 = orc.sparse_decode_attn_fp8(q, k8, v8, ks, vs, idx, N)
    o16, l16, _ = orc.sparse_decode_attn(q, k16, v16, idx, N)
    np.testing.assert_allclose(o8, o16, atol=1e-12)
    np.testing.assert_allclose(l8, l16, atol=1e-12)
    # scaling V by 2^-3 scales the output exactly
    v8b, vsb = orc.quantize_fp8(bf(v * 2.0 ** -3), N)
    np.testing.assert_array_equal(v8b, v8)
    o8b, _ = orc.sparse_decode_attn_fp8(q, k8, v8b, ks, vsb, idx, N)
    np.testing.assert_allclose(o8b, o8 * 2.0 ** -3, atol=1e-12)


def test_fp8_attention_applies_each_blocks_scales(orc):
    # the representable cache above with block j's keys times 2^-(j+1) and its values times
    # 2^(j-2): each block quantizes to exactly that scale and the same codes, so the
    # attention of the FP8 cache must equal the bf16 attention of the scaled values
    # (the key scale enters every logit of its block, the value scale every value row)
    rng = np.random.default_rng(44)
    fin = np.array(sorted({orc.e4m3_value(c) for c in range(0, 127)}))
    pool = np.concatenate([fin[(fin > 0.05) & (fin < 4)], -fin[(fin > 0.05) & (fin < 4)]])
    B, Hq, Hkv, d, nb = 1, 4, 2, 16, 6
    N = 64 * nb - 9
    k = rng.choice(pool, (B, Hkv, N, d)).astype(np.float32)
    v = rng.choice(pool, (B, Hkv, N, d)).astype(np.float32)
    for j in range(nb):
        k[:, :, j * 64, 0] = 448.0
        v[:, :, j * 64, 1] = 448.0
        k[:, :, j * 64:(j + 1) * 64] *= 2.0 ** -(j + 1)
        v[:, :, j * 64:(j + 1) * 64] *= 2.0 ** (j - 2)
    q = bf(rng.standard_normal((B, Hq, d)).astype(np.float32) * 0.5)
    k16, v16 = bf(k), bf(v)
    assert np.array_equal(f(k16), k) and np.array_equal(f(v16), v)
    k8, ks = orc.quantize_fp8(k16, N)
    v8, vs = orc.quantize_fp8(v16, N)
    np.testing.assert_array_equal(ks[0, 0], 2.0 ** -(np.arange(nb) + 1))
    np.testing.assert_array_equal(vs[0, 1], 2.0 ** (np.arange(nb) - 2))
    idx = np.array([[[0, 1, 3, 5], [0, 2, 4, 5]]], np.int32)
    o8, l8 = orc.sparse_decode_attn_fp8(q, k8, v8, ks, vs, idx, N)
    o16, l16, _ = orc.sparse_decode_attn(q, k16, v16, idx, N)
    np.testing.assert_allclose(o8, o16, atol=1e-12)
    np.testing.assert_allclose(l8, l16, atol=1e-12)
    # the scales differ enough that a dropped or misplaced key scale would show
    ku, _ = orc.quantize_fp8(bf(k * (2.0 ** (np.arange(N) // 64 + 1))[None, None, :, None]), N)
    np.testing.assert_array_equal(ku, k8)
    o_unscaled, _, _ = orc.sparse_decode_attn(
        q, bf(k * (2.0 ** (np.arange(N) // 64 + 1))[None, None, :, None]), v16, idx, N)
    assert np.abs(o_unscaled - o16).max() > 1e-3
