"""GPU parity of the chunked-prefill path (streams, tile selection, three branches) vs the oracle.

Every case prints its name, seed and shapes before touching the GPU.
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


def check_tile_selection(g_sel, o_sel, o_scores, rel=TIE_REL):
    """Per (b, tile, kvh): equal sets, or differences only at near-ties of the k-th score."""
    exempt = 0
    B, T, H, k = g_sel.shape
    for b in range(B):
        for t in range(T):
            for h in range(H):
                g, o = g_sel[b, t, h], o_sel[b, t, h]
                assert len(g) == len(o) == k, (b, t, h)
                assert g.min() >= 0 and g.max() < o_scores.shape[-1], (b, t, h)
                assert np.all(np.diff(g) > 0), (b, t, h)
                if np.array_equal(g, o):
                    continue
                sc = o_scores[b, t, h]
                tau = sc[o].min()
                for j in set(g.tolist()) ^ set(o.tolist()):
                    assert abs(sc[j] - tau) <= rel * max(abs(sc[j]), abs(tau)), (b, t, h, j)
                    exempt += 1
    return exempt


def run_prefill_case(cfg, seed, rows=None, combine=0, sink=None, indexer=bsa.INDEXER_BF16):
    import torch
    announce(cfg.name, "seed", seed, "B", cfg.batch, "Hq", cfg.n_q_heads, "Hkv", cfg.n_kv_heads,
             "P", cfg.prior_len, "C", cfg.chunk_len, "m", cfg.m_sparse, cfg.m_dense, "top_k",
             cfg.top_k_sparse, "window", cfg.window, "q_tile", cfg.q_tile, "combine", combine,
             "sink", None if sink is None else list(np.round(sink, 3)), "indexer", indexer)
    t = synth.gen_prefill(cfg, seed)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    pc = bsa.prefill_cfg(cfg.m_sparse, cfg.top_k_sparse, cfg.m_dense, cfg.window, cfg.q_tile,
                         combine, indexer=indexer)
    sink_dev = None if sink is None else torch.from_numpy(
        np.asarray(sink, np.float32)).to(q.device)
    out, lse3, sel = bsa.prefill_step(q, k, v, cfg.prior_len, pc, want_lse3=True, want_sel=True,
                                      sink_logits=sink_dev)
    torch.cuda.synchronize()
    g_out, g_lse3, g_sel = out.cpu().numpy(), lse3.cpu().numpy(), sel.cpu().numpy()
    common = dict(m_sparse=cfg.m_sparse, top_k=cfg.top_k_sparse, m_dense=cfg.m_dense,
                  window=cfg.window, q_tile=cfg.q_tile)
    ref_sel = oracle.sparse_prefill_attn(t["q"], t["k"], t["v"], cfg.prior_len, rows=[0],
                                         want_sel=True, want_sel_scores=True, indexer=indexer,
                                         **common)
    exempt = check_tile_selection(g_sel, ref_sel["sel"], ref_sel["sel_scores"])
    ref = oracle.sparse_prefill_attn(t["q"], t["k"], t["v"], cfg.prior_len, sel_in=g_sel,
                                     rows=rows, combine=combine,
                                     sink_logits=None if sink is None
                                     else np.asarray(sink, np.float32).astype(np.float64),
                                     **common)
    gsub = g_out if rows is None else g_out[:, rows]
    lsub = g_lse3 if rows is None else g_lse3[:, :, rows]
    err = np.abs(gsub - ref["out"]).max()
    lerr = np.abs(lsub - ref["lse3"]).max()
    announce("  exempt ties", exempt, "max|out err|", err, "max|lse err|", lerr)
    assert np.isfinite(gsub).all()
    assert err <= OUT_ATOL, err
    assert lerr <= 1e-3, lerr
    return err


def small(**kw):
    base = dict(name="pf_small", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128,
                prior_len=64 * 40 + 16, chunk_len=100, top_k_sparse=96, window=128)
    base.update(kw)
    return synth.PrefillConfig(**base)


def test_compressed_streams_bit_exact():
    """The pooled streams (m = 4 fp32 + bf16 keys, bf16 values; m = 128 bf16 keys and values)
    over a ragged prior length equal the oracle's fp32 token-order means and their bf16
    roundings bit for bit."""
    import torch
    cfg = small(name="pf_streams", prior_len=64 * 37 + 22)
    announce(cfg.name, "seed", 71, "P", cfg.prior_len, "streams")
    t = synth.gen_prefill(cfg, 71)
    k, v = to_dev(t["k"]), to_dev(t["v"])
    pc = bsa.prefill_cfg(cfg.m_sparse, cfg.top_k_sparse, cfg.m_dense, cfg.window, cfg.q_tile)
    k4f, k4b, v4b, k128b, v128b = bsa.build_compressed_streams(k, v, cfg.prior_len, pc,
                                                                want_f32=True)
    torch.cuda.synchronize()
    bits = lambda a: a.view(torch.int16).cpu().numpy().view(np.uint16)
    rne = np.vectorize(oracle.round_bf16, otypes=[np.uint16])
    P = cfg.prior_len
    o_k4 = oracle.block_summaries_f32(t["k"], P, cfg.m_sparse)
    assert np.array_equal(k4f.cpu().numpy(), o_k4)
    assert np.array_equal(bits(k4b), rne(o_k4.astype(np.float64)))
    for got, x, m in ((v4b, t["v"], cfg.m_sparse), (k128b, t["k"], cfg.m_dense),
                      (v128b, t["v"], cfg.m_dense)):
        o = oracle.block_summaries_f32(x, P, m)
        assert np.array_equal(bits(got), rne(o.astype(np.float64))), m


def test_streams_and_selection_with_cancelling_sums():
    """Keys whose 4-token groups hold 2^20 and -2^20 around a small value in some dims: the
    fp32 running sums lose that value's low bits, so the pooled keys differ from the
    rounded exact means.  The GPU's streams equal the oracle's fp32 token-order means and
    their bf16 roundings bit for bit, and the selection against those bf16 keys matches
    the oracle's (near-tie rule)."""
    import torch
    cfg = small(name="pf_cancel", prior_len=64 * 60 + 9, chunk_len=70, top_k_sparse=200)
    seed = 79
    announce(cfg.name, "seed", seed, "P", cfg.prior_len, "cancelling pairs")
    t = synth.gen_prefill(cfg, seed)
    k = synth.bf16_to_f32(t["k"]).copy()
    rng = np.random.default_rng(seed)
    n_grp = cfg.prior_len // 4
    grp = rng.choice(n_grp, n_grp // 3, replace=False)
    dims = rng.choice(128, 16, replace=False)
    for j in grp:
        k[:, :, 4 * j, dims] = 2.0 ** 20
        k[:, :, 4 * j + 2, dims] = -(2.0 ** 20)
    t["k"] = synth.bf16_round(k)
    q, kd, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    pc = bsa.prefill_cfg(cfg.m_sparse, cfg.top_k_sparse, cfg.m_dense, cfg.window, cfg.q_tile)
    st = bsa.build_compressed_streams(kd, v, cfg.prior_len, pc, want_f32=True)
    sel = bsa.select_prefill_entries(q, kd, None, st[1], cfg.prior_len, cfg=pc)
    torch.cuda.synchronize()
    o_k4 = oracle.block_summaries_f32(t["k"], cfg.prior_len, cfg.m_sparse)
    exact = oracle.block_summaries(t["k"], cfg.prior_len, cfg.m_sparse)
    assert not np.array_equal(o_k4.astype(np.float64), exact)  # the fp32 sums did round
    assert np.array_equal(st[0].cpu().numpy(), o_k4)
    rne = np.vectorize(oracle.round_bf16, otypes=[np.uint16])
    assert np.array_equal(st[1].view(torch.int16).cpu().numpy().view(np.uint16),
                          rne(o_k4.astype(np.float64)))
    ref = oracle.sparse_prefill_attn(t["q"], t["k"], t["v"], cfg.prior_len, rows=[0],
                                     m_sparse=cfg.m_sparse, top_k=cfg.top_k_sparse,
                                     m_dense=cfg.m_dense, window=cfg.window,
                                     q_tile=cfg.q_tile, want_sel=True, want_sel_scores=True)
    announce("  exempt ties", check_tile_selection(sel.cpu().numpy(), ref["sel"],
                                                   ref["sel_scores"]))


@pytest.mark.parametrize("indexer", [bsa.INDEXER_BF16, bsa.INDEXER_F32])
def test_prefill_small_ragged_g4(indexer):
    run_prefill_case(small(), 61, indexer=indexer)


@pytest.mark.parametrize("chunk_len", [645, 1000])
@pytest.mark.parametrize("indexer", [bsa.INDEXER_BF16, bsa.INDEXER_F32])
def test_prefill_many_tiles(chunk_len, indexer):
    """Tiles of 16 queries (x 4 heads): 41 and 63 tiles, so the scores kernels hold three
    and four blocks of 16 tiles' pooled queries (the last one partial), over a ragged
    3,001-entry stream; 40 sampled rows."""
    cfg = small(name=f"pf_tiles{chunk_len}", prior_len=4 * 3001 - 2, chunk_len=chunk_len,
                q_tile=16, top_k_sparse=300, window=40)
    rows = np.sort(np.random.default_rng(chunk_len).choice(chunk_len, 40, replace=False))
    run_prefill_case(cfg, 63 + indexer, rows=rows, indexer=indexer)


@pytest.mark.parametrize("g", [1, 2])
def test_prefill_small_groups(g):
    run_prefill_case(small(name=f"pf_g{g}", n_q_heads=2 * g, batch=2), 62 + g)


def test_prefill_window_and_topk_edges():
    # window longer than the whole context; top-k covering every entry
    run_prefill_case(small(name="pf_bigwin", window=10_000, top_k_sparse=10_000), 71)
    # window of one token (the query itself); top-1
    run_prefill_case(small(name="pf_win1", window=1, top_k_sparse=1, chunk_len=70), 72)
    # small prior context (fewer entries than top-k), partial dense entry
    run_prefill_case(small(name="pf_tiny_prior", prior_len=300, chunk_len=64), 73)


@pytest.mark.parametrize("g", [4, 2])
def test_prefill_largest_selection(g):
    """The largest branch-A selection the attention keeps in LDS (4,096 entries) out of 5,003,
    for 256- and 128-row tiles."""
    run_prefill_case(small(name=f"pf_maxsel_g{g}", n_q_heads=2 * g, prior_len=4 * 5003,
                           chunk_len=90, top_k_sparse=4096), 74 + g)


@pytest.mark.parametrize("prior_len,indexer", [(400_000, bsa.INDEXER_BF16),
                                               (400_000, bsa.INDEXER_F32),
                                               (524_288, bsa.INDEXER_BF16)])
def test_prefill_long_prior_wide_topk(prior_len, indexer):
    """Prior contexts of 400,000 and 524,288 tokens: 100,000 and 131,072 (the most the
    selection supports) m = 4 entries per kv head, so the selection takes the 1024-thread
    top-k and branch A gathers entries past 2^16; 3 tiles, 24 sampled rows."""
    cfg = small(name=f"pf_long_prior{prior_len}", prior_len=prior_len, chunk_len=130,
                top_k_sparse=2048)
    rows = np.sort(np.random.default_rng(400).choice(130, 24, replace=False))
    run_prefill_case(cfg, 401, rows=rows, indexer=indexer)


@pytest.mark.parametrize("combine,with_sink", [(1, False), (0, True), (1, True)])
def test_prefill_combine_and_sink(combine, with_sink):
    # concatenated softmax over the branches ("CSA + HCA 混合注意力机制" §4.3) and per-head
    # sink logits (§5.4); sinks span below, near and above the rows' lse values
    cfg = small(name=f"pf_comb{combine}{'s' if with_sink else ''}", n_q_heads=8)
    sink = np.linspace(-4.0, 6.0, cfg.n_q_heads) if with_sink else None
    run_prefill_case(cfg, 91 + combine, combine=combine, sink=sink)


def test_prefill_full_size_concat_sink_sampled_rows():
    cfg = synth.CONFIGS["prefill256k"]
    rows = np.array([0, 64, 777, 2047])
    sink = np.linspace(-2.0, 3.0, cfg.n_q_heads)
    run_prefill_case(cfg, synth.DEFAULT_SEED["prefill256k"], rows=rows, combine=1, sink=sink)


def test_prefill_full_size_sampled_rows():
    cfg = synth.CONFIGS["prefill256k"]
    rows = np.array([0, 1, 63, 64, 500, 1023, 1024, 1500, 2046, 2047])
    run_prefill_case(cfg, synth.DEFAULT_SEED["prefill256k"], rows=rows)


def test_prefill_full_size_two_whole_tiles():
    """Every query row and head of the first and the last tile (64 queries x 32 heads each)
    of the 262K workload."""
    cfg = synth.CONFIGS["prefill256k"]
    rows = np.r_[0:64, 1984:2048]
    run_prefill_case(cfg, synth.DEFAULT_SEED["prefill256k"], rows=rows)


@pytest.mark.parametrize("indexer", [bsa.INDEXER_BF16, bsa.INDEXER_F32])
def test_prefill_full_size_second_seed(indexer):
    cfg = synth.CONFIGS["prefill256k"]
    rows = np.array([0, 5, 63, 64, 130, 999, 1024, 1535, 1536, 2047])
    run_prefill_case(cfg, 105, rows=rows, indexer=indexer)


def test_prefill_values_near_the_fp16_limit():
    """P V runs on the fp16 matrix cores, so values must lie inside fp16's range (|v| <=
    65504).  V times 2^13 (|v| up to ~37,000, every bf16 value still exact) stays in range: the
    outputs scale by 2^13 and the error bound with them (it is relative to the values)."""
    import torch
    cfg = small(name="pf_bigv", chunk_len=70)
    seed = 77
    scale = 2.0 ** 13
    announce(cfg.name, "seed", seed, "V x", scale)
    t = synth.gen_prefill(cfg, seed)
    v_big = synth.bf16_round(synth.bf16_to_f32(t["v"]) * np.float32(scale))
    assert np.array_equal(synth.bf16_to_f32(v_big), synth.bf16_to_f32(t["v"]) * scale)
    vmax = float(np.abs(synth.bf16_to_f32(v_big)).max())
    assert 30000 < vmax <= 65504, vmax
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(v_big)
    pc = bsa.prefill_cfg(cfg.m_sparse, cfg.top_k_sparse, cfg.m_dense, cfg.window, cfg.q_tile)
    out, lse3, sel = bsa.prefill_step(q, k, v, cfg.prior_len, pc, want_lse3=True, want_sel=True)
    torch.cuda.synchronize()
    common = dict(m_sparse=cfg.m_sparse, top_k=cfg.top_k_sparse, m_dense=cfg.m_dense,
                  window=cfg.window, q_tile=cfg.q_tile)
    ref = oracle.sparse_prefill_attn(t["q"], t["k"], v_big, cfg.prior_len,
                                     sel_in=sel.cpu().numpy(), **common)
    g = out.cpu().numpy()
    err = np.abs(g - ref["out"]).max()
    announce("  max|out err|", err, "max|out|", np.abs(ref["out"]).max())
    assert np.isfinite(g).all()
    assert err <= OUT_ATOL * scale, err
    assert np.abs(lse3.cpu().numpy() - ref["lse3"]).max() <= 1e-3


@pytest.mark.parametrize("indexer", [bsa.INDEXER_BF16, bsa.INDEXER_F32])
def test_prefill_split_entry_points_compose(indexer):
    """select_prefill_entries + sparse_prefill_attn_selected equal sparse_prefill_attn bit for
    bit; the attention step alone matches the oracle on the oracle's own selection; selection
    indices out of range are clamped (memory-safe) like an explicitly clamped list."""
    import torch
    cfg = small(name="pf_split", batch=2, chunk_len=130)
    seed = 81
    announce(cfg.name, "seed", seed, "split entry points", "indexer", indexer)
    t = synth.gen_prefill(cfg, seed)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    pc = bsa.prefill_cfg(cfg.m_sparse, cfg.top_k_sparse, cfg.m_dense, cfg.window, cfg.q_tile,
                         indexer=indexer)
    st = bsa.build_compressed_streams(k, v, cfg.prior_len, pc)
    out, _, sel = bsa.sparse_prefill_attn(q, k, v, *st, cfg.prior_len, cfg=pc, want_sel=True)
    sel2 = bsa.select_prefill_entries(q, k, st[0], st[1], cfg.prior_len, cfg=pc)
    out2, _ = bsa.sparse_prefill_attn_selected(q, k, v, *st[1:], sel2, cfg.prior_len, cfg=pc)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel2)
    assert torch.equal(out, out2)
    common = dict(m_sparse=cfg.m_sparse, top_k=cfg.top_k_sparse, m_dense=cfg.m_dense,
                  window=cfg.window, q_tile=cfg.q_tile)
    o_sel = oracle.sparse_prefill_attn(t["q"], t["k"], t["v"], cfg.prior_len, rows=[0],
                                       want_sel=True, indexer=indexer, **common)["sel"]
    ref = oracle.sparse_prefill_attn(t["q"], t["k"], t["v"], cfg.prior_len, sel_in=o_sel,
                                     **common)
    out3, lse3 = bsa.sparse_prefill_attn_selected(q, k, v, *st[1:],
                                                  torch.from_numpy(o_sel).to(q.device),
                                                  cfg.prior_len, cfg=pc, want_lse3=True)
    torch.cuda.synchronize()
    err = np.abs(out3.cpu().numpy() - ref["out"]).max()
    lerr = np.abs(lse3.cpu().numpy() - ref["lse3"]).max()
    announce("  oracle selection: max|out err|", err, "max|lse err|", lerr)
    assert err <= OUT_ATOL and lerr <= 1e-3
    e_s = bsa.num_blocks(cfg.prior_len, cfg.m_sparse)
    wild = sel2.clone()
    wild[..., -1] = e_s + 1000
    wild[..., 0] = -7
    tame = wild.clamp(0, e_s - 1)
    o_w, _ = bsa.sparse_prefill_attn_selected(q, k, v, *st[1:], wild, cfg.prior_len, cfg=pc)
    o_t, _ = bsa.sparse_prefill_attn_selected(q, k, v, *st[1:], tame, cfg.prior_len, cfg=pc)
    torch.cuda.synchronize()
    assert torch.equal(o_w, o_t)


@pytest.mark.parametrize("indexer", [bsa.INDEXER_BF16, bsa.INDEXER_F32])
@pytest.mark.parametrize("prior_len", [64 * 40 + 16, 160_000, 270_000])
def test_prefill_selection_exact_ties(prior_len, indexer):
    """Integer keys constant over every 4-token group and integer queries: the pooled m = 4
    keys are exact, the fp32 scores exact integers with many equal values, so the tile
    selection must equal the oracle's exactly (lower entry index first at the k-th score).
    Covers the top-k's tie path at 4 (644 entries) and 128 keys per thread with 512 threads
    (40,000 entries) and with 1024 threads (67,500 entries); random scores (the other tests)
    take the path without ties."""
    import torch
    B, Hq, Hkv, d, C, top_k = 1, 4, 1, 128, 64, 96
    announce("pf_ties", "P", prior_len, "top_k", top_k, "indexer", indexer)
    rng = np.random.default_rng(prior_len)
    n_tok = prior_len + C
    groups = rng.integers(-2, 3, (B, Hkv, -(-n_tok // 4), d)).astype(np.float32)
    k = synth.bf16_round(np.repeat(groups, 4, axis=2)[:, :, :n_tok])
    v = synth.bf16_round(rng.standard_normal((B, Hkv, n_tok, d)).astype(np.float32))
    q = synth.bf16_round(rng.integers(-1, 2, (B, C, Hq, d)).astype(np.float32))
    pc = bsa.prefill_cfg(4, top_k, 128, 128, 64, indexer=indexer)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    st = bsa.build_compressed_streams(kd, vd, prior_len, pc)
    sel = bsa.select_prefill_entries(qd, kd, st[0], st[1], prior_len, cfg=pc)
    torch.cuda.synchronize()
    o_sel = oracle.sparse_prefill_attn(q, k, v, prior_len, m_sparse=4, top_k=top_k, m_dense=128,
                                       window=128, q_tile=64, rows=[0], want_sel=True,
                                       indexer=indexer)["sel"]
    g_sel = sel.cpu().numpy()
    assert g_sel.shape == o_sel.shape
    assert np.array_equal(g_sel, o_sel)


@pytest.mark.parametrize("prior_len,top_k,keys", [
    (80_000, 96, "equal"),    # 20,000 equal scores: the sample's bracket holds more keys than
                              # the top-k stages, so the bit passes run (nothing above the
                              # undecided range)
    (40_000, 96, "equal"),    # 10,000 equal scores: staged, the bracket is the largest key
    (8_192, 1_024, "normal"),  # k / entries = 1/2: no sample rank brackets it; all 2,048 keys
                              # fit the staging, so no bit pass runs and the radix digits fix T
    (64 * 700, 600, "normal"),  # 11,200 entries, a bracketed sample
    (64 * 700 + 12, 600, "normal"),  # 11,203 entries: a ragged last float4 of the row
])
def test_prefill_selection_threshold_paths(prior_len, top_k, keys):
    """The tile selection equals the oracle's on inputs that steer the top-k's threshold
    search down each of its paths (sample bracket, every key staged, bit passes) and through
    all-equal scores, where the lowest entry indices are taken."""
    _threshold_case(prior_len, top_k, keys)


@pytest.mark.parametrize("prior_len,top_k,keys", [(64 * 700 + 12, 600, "normal"),
                                                  (40_000, 96, "equal")])
def test_prefill_selection_threshold_batched(prior_len, top_k, keys):
    """The same over 2 batch entries x 2 kv heads x 2 tiles: every (batch, tile, kv head)
    row finds its own threshold and writes its own selection."""
    _threshold_case(prior_len, top_k, keys, B=2, Hkv=2, Hq=8, C=128)


@pytest.mark.parametrize("n_entries", [30_000, 70_000])
def test_prefill_selection_distinct_tops_over_ties(n_entries):
    """40 distinct high scores above tens of thousands of equal ones, k = 96: the sample's
    bracket is the common value and holds more keys than the top-k stages, so the bit passes
    run with the 40 distinct keys above the undecided range, then the digits and the
    emission from the registers.  30,000 entries take the 512-thread variant, 70,000 the
    1024-thread one.  Exact scores: the selection must equal the oracle's (the 40, then the
    56 lowest indices of the equal entries)."""
    _distinct_over_ties(4 * n_entries, 96, n_high=40, seed=n_entries)


def test_prefill_selection_sparse_high_scores_over_ties():
    """512 high scores on every 40th of 20,480 entries and equal low scores elsewhere,
    k = 1,024: the threshold lies among the equal scores, so the selection is the 512 high
    entries and the 512 lowest-index low ones (the bit passes run with the high keys above
    the undecided range)."""
    E = 20_480
    high = (np.arange(512) * E) // 512
    _distinct_over_ties(4 * E, 1_024, high_at=high, seed=5)


@pytest.mark.parametrize("n_entries,n_mid", [(30_000, 4_000), (70_000, 8_000)])
def test_prefill_selection_tied_threshold_bucket(n_entries, n_mid):
    """40 distinct high scores, n_mid equal middle scores above equal low ones, k = 540: the
    sample's bracket is the middle value, so the top-k stages the high and middle keys, and
    the value bucket holding the k-th largest key holds every middle key (more than the 256
    it ranks directly): radix digits over the staged keys fix T.  30,000 entries take the
    512-thread variant, 70,000 the 1024-thread one (a CPU replay of the kernel's decisions
    on these inputs: 4,040 and 8,040 keys staged).  Exact scores: the selection must equal
    the oracle's (the 40, then the 500 lowest-index middle entries)."""
    _distinct_over_ties(4 * n_entries, 540, n_high=40, n_mid=n_mid, seed=n_entries + 1)


def _distinct_over_ties(prior_len, top_k, n_high=0, high_at=None, seed=0, n_mid=0):
    import torch
    d, C, Hq = 128, 64, 4
    E = prior_len // 4
    announce("pf_tops", "P", prior_len, "E", E, "top_k", top_k, "high", n_high,
             "high_at", None if high_at is None else len(high_at), "mid", n_mid)
    rng = np.random.default_rng(seed)
    n_tok = prior_len + C
    # every 4-token group pools to ones (score 256 * 128 with q = ones), except the high
    # entries, whose dim 0 is 2 + r / 4 (distinct, exact in bf16), and n_mid middle entries
    # (dim 0 = 1.5: one score between the two)
    k = np.ones((1, 1, n_tok, d), np.float32)
    pos = rng.choice(E, n_high, replace=False) if high_at is None else np.asarray(high_at)
    for r, j in enumerate(pos):
        k[0, 0, 4 * j:4 * j + 4, 0] = 2.0 + 0.25 * (r % 40) + 16.0 * (r // 40)
    if n_mid:
        mid = rng.choice(np.setdiff1d(np.arange(E), pos), n_mid, replace=False)
        for j in mid:
            k[0, 0, 4 * j:4 * j + 4, 0] = 1.5
    k = synth.bf16_round(k)
    v = synth.bf16_round(rng.standard_normal((1, 1, n_tok, d)).astype(np.float32))
    q = synth.bf16_round(np.ones((1, C, Hq, d), np.float32))
    pc = bsa.prefill_cfg(4, top_k, 128, 128, 64)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    st = bsa.build_compressed_streams(kd, vd, prior_len, pc)
    sel = bsa.select_prefill_entries(qd, kd, st[0], st[1], prior_len, cfg=pc)
    torch.cuda.synchronize()
    o_sel = oracle.sparse_prefill_attn(q, k, v, prior_len, m_sparse=4, top_k=top_k, m_dense=128,
                                       window=128, q_tile=64, rows=[0], want_sel=True)["sel"]
    g_sel = sel.cpu().numpy()
    assert g_sel.shape == o_sel.shape
    assert np.array_equal(g_sel, o_sel)
    assert set(pos.tolist()) <= set(o_sel.reshape(-1).tolist())


def _threshold_case(prior_len, top_k, keys, B=1, Hkv=1, Hq=4, C=64):
    import torch
    d = 128
    announce("pf_thr", "B", B, "Hkv", Hkv, "P", prior_len, "top_k", top_k, keys)
    rng = np.random.default_rng(prior_len + top_k + B)
    n_tok = prior_len + C
    if keys == "equal":
        k = synth.bf16_round(np.ones((B, Hkv, n_tok, d), np.float32))
        q = synth.bf16_round(rng.integers(-1, 2, (B, C, Hq, d)).astype(np.float32))
    else:
        k = synth.bf16_round(rng.standard_normal((B, Hkv, n_tok, d)).astype(np.float32))
        q = synth.bf16_round(rng.standard_normal((B, C, Hq, d)).astype(np.float32))
    v = synth.bf16_round(rng.standard_normal((B, Hkv, n_tok, d)).astype(np.float32))
    pc = bsa.prefill_cfg(4, top_k, 128, 128, 64)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    st = bsa.build_compressed_streams(kd, vd, prior_len, pc)
    sel = bsa.select_prefill_entries(qd, kd, st[0], st[1], prior_len, cfg=pc)
    torch.cuda.synchronize()
    ref = oracle.sparse_prefill_attn(q, k, v, prior_len, m_sparse=4, top_k=top_k, m_dense=128,
                                     window=128, q_tile=64, rows=[0], want_sel=True,
                                     want_sel_scores=True)
    o_sel = ref["sel"]
    g_sel = sel.cpu().numpy()
    assert g_sel.shape == o_sel.shape
    if keys == "equal":
        assert np.array_equal(o_sel.reshape(-1, top_k)[0], np.arange(top_k))
        assert np.array_equal(g_sel, o_sel)
    else:
        announce("  exempt ties", check_tile_selection(g_sel, o_sel, ref["sel_scores"]))
