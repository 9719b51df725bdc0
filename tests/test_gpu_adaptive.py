"""GPU parity of the anchor-adaptive selection (k per (b, kv head) from the sink
and local anchors' scores, lists padded with -1) and of decode attention over
padded lists, against the oracle.

Every case prints its name, seed and sizes before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import long_context_block_summary_amd as bsa
from long_context_block_summary_amd import synth
from parity_rules import OUT_ATOL, TIE_REL, to_dev

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


def oracle_topk(sc, c0, c1, k):
    """Indices of the k highest candidate scores, lower index first on ties."""
    cand = np.arange(c0, c1)
    order = np.lexsort((cand, -sc[c0:c1]))
    return cand[order[:k]]


def run_adaptive(name, seed, B, Hq, Hkv, d, N, rmin, rmax, margin):
    import torch
    announce(name, "seed", seed, "B", B, "Hq", Hq, "Hkv", Hkv, "d", d, "N", N, "range", rmin,
             rmax, "margin", margin)
    cfg = synth.DecodeConfig(name=name, batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                             seq_len=N)
    t = synth.gen_decode(cfg, seed)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    bs, nb = 64, -(-N // 64)
    summ, _ = bsa.build_block_summaries(k, N, bs)
    idx, scores = bsa.select_blocks(q, summ, N, bs, 1, 2, -1, rmin, want_scores=True,
                                    adaptive=True, keep_ratio_max=rmax, anchor_margin=margin)
    out, lse = bsa.sparse_decode_attn(q, k, v, idx, N, bs)
    torch.cuda.synchronize()
    g_idx, g_sc = idx.cpu().numpy(), scores.cpu().numpy()
    o_summ = oracle.block_summaries(t["k"], N, bs)
    o_idx, o_cnt, o_sc = oracle.select_blocks_adaptive(t["q"], o_summ, Hkv, 1, 2, rmin, rmax,
                                                       margin)
    width, k_lo, k_hi = oracle.adaptive_bounds(nb, 1, 2, rmin, rmax)
    assert g_idx.shape[2] == width
    c0, c1 = 1, nb - 2
    flips, counts = 0, []
    for b in range(B):
        for h in range(Hkv):
            row = g_idx[b, h]
            cnt = int((row >= 0).sum())
            assert (row[:cnt] >= 0).all() and (row[cnt:] == -1).all(), "padding not at the end"
            assert np.all(np.diff(row[:cnt]) > 0)
            kk = cnt - 3
            assert k_lo <= kk <= k_hi
            counts.append(cnt)
            sc = o_sc[b, h]
            anchors = np.r_[sc[:c0], sc[c1:]]
            a_max, a_min = anchors.max(), anchors.min()
            tau = a_max + margin * (a_max - a_min)
            if cnt != o_cnt[b, h]:
                # only candidates within the fp32 decision's reach of tau may flip
                tol = TIE_REL * max(abs(a_max), abs(a_min), abs(tau), 1e-30) * (1 + abs(margin))
                lo = int((sc[c0:c1] > tau + tol).sum())
                hi = int((sc[c0:c1] > tau - tol).sum())
                assert min(max(lo, k_lo), k_hi) <= kk <= min(max(hi, k_lo), k_hi), (b, h, cnt)
                flips += 1
            # the kept set is the top-kk of the candidates (near-tie rule at the k-th score)
            got = set(row[:cnt].tolist()) - {0, nb - 2, nb - 1}
            want = set(oracle_topk(sc, c0, c1, kk).tolist())
            assert {0, nb - 2, nb - 1} <= set(row[:cnt].tolist())
            if got != want:
                kth = sc[list(want)].min() if want else 0.0
                for j in got ^ want:
                    assert abs(sc[j] - kth) <= TIE_REL * max(abs(sc[j]), abs(kth)), (b, h, j)
    # scores of every block (anchors included) against the oracle's
    np.testing.assert_allclose(g_sc, o_sc, rtol=1e-4, atol=1e-3 * np.abs(o_sc).max())
    o_out, o_lse, _ = oracle.sparse_decode_attn(t["q"], t["k"], t["v"], g_idx, N, bs)
    err = float(np.abs(out.cpu().numpy() - o_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - o_lse).max())
    announce("  kept per pair", counts, "count flips", flips, "max|out err|", err)
    assert err <= OUT_ATOL and lerr <= 1e-3
    return counts


@pytest.mark.parametrize("margin", [0.0, 0.5, -0.3])
def test_adaptive_selection_and_attention(margin):
    counts = run_adaptive(f"adapt_m{margin}", 51, B=2, Hq=8, Hkv=4, d=128, N=64 * 150 + 37,
                          rmin=0.1, rmax=0.3, margin=margin)
    assert len(set(counts)) >= 1


def test_adaptive_extremes_and_groups():
    # a huge margin keeps the minimum everywhere, a very negative one the maximum
    w, k_lo, k_hi = oracle.adaptive_bounds(-(-(64 * 90 + 1) // 64), 1, 2, 0.1, 0.2)
    c = run_adaptive("adapt_min", 52, B=1, Hq=16, Hkv=1, d=128, N=64 * 90 + 1, rmin=0.1,
                     rmax=0.2, margin=1e6)
    assert all(x == 3 + k_lo for x in c)
    c = run_adaptive("adapt_max", 53, B=2, Hq=4, Hkv=2, d=64, N=64 * 90 + 1, rmin=0.1,
                     rmax=0.2, margin=-1e6)
    assert all(x == 3 + k_hi for x in c)
    # the 128K workload's shapes, keep range 10-20 %
    run_adaptive("adapt_128k", 3, B=4, Hq=64, Hkv=8, d=128, N=131072, rmin=0.1, rmax=0.2,
                 margin=0.0)
