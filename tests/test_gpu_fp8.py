"""GPU parity of the FP8 (OCP E4M3) KV cache: quantize_kv_fp8 must write the
oracle's codes and scales bit for bit; sparse_decode_attn_fp8 must match the
oracle's attention over the dequantized cache (the oracle's own codes are
uploaded, so the attention check does not lean on the quantizer).

Every case prints its name, seed and sizes before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import long_context_block_summary_amd as bsa
from long_context_block_summary_amd import synth
from parity_rules import OUT_ATOL, to_dev

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


@pytest.mark.parametrize("d,N,cap", [(128, 64 * 40 + 17, 64 * 44), (64, 64 * 9, 64 * 9)])
def test_quantize_matches_oracle_bit_for_bit(d, N, cap):
    import torch
    announce("quantize", "d", d, "N", N, "capacity", cap)
    rng = np.random.default_rng(d + N)
    x = rng.standard_normal((2, 3, cap, d)).astype(np.float32) * np.exp2(rng.integers(-20, 12))
    x[0, 1, 64:128] = 0.0                      # an all-zero block
    x[1, 2, 5, 7] = 3.0e4                      # one large outlier in a block
    x16 = synth.bf16_round(x)
    o_codes, o_sc = oracle.quantize_fp8(x16, N, 64, sstride=cap // 64)
    codes, sc = bsa.quantize_kv_fp8(to_dev(x16), N, 64, summary_stride=cap // 64)
    torch.cuda.synchronize()
    g_codes, g_sc = codes.cpu().numpy(), sc.cpu().numpy()
    nb = -(-N // 64)
    assert np.array_equal(g_sc[..., :nb].view(np.uint32), o_sc[..., :nb].view(np.uint32))
    assert np.array_equal(g_codes[:, :, :N], o_codes[:, :, :N])
    assert not g_codes[:, :, N:].any()         # rows past seq_len untouched (zero-filled here)


def run_fp8_decode(name, seed, cfg, adaptive=False):
    import torch
    announce(name, "seed", seed, "B", cfg.batch, "Hq", cfg.n_q_heads, "Hkv", cfg.n_kv_heads,
             "d", cfg.head_dim, "N", cfg.seq_len, "top_k", cfg.top_k, "adaptive", adaptive)
    t = synth.gen_decode(cfg, seed)
    N, bs = cfg.seq_len, cfg.block_size
    q, k = to_dev(t["q"]), to_dev(t["k"])
    k8, ks = oracle.quantize_fp8(t["k"], N, bs)
    v8, vs = oracle.quantize_fp8(t["v"], N, bs)
    summ, _ = bsa.build_block_summaries(k, N, bs)
    kw = dict(adaptive=True, keep_ratio_max=0.3) if adaptive else {}
    idx, _ = bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k,
                               0.1 if adaptive else cfg.keep_ratio, **kw)
    dev = q.device
    tt = lambda a: torch.from_numpy(a).to(dev)
    out, lse = bsa.sparse_decode_attn_fp8(q, tt(k8), tt(v8), tt(ks), tt(vs), idx, N, bs)
    torch.cuda.synchronize()
    g_idx = idx.cpu().numpy()
    o_out, o_lse = oracle.sparse_decode_attn_fp8(t["q"], k8, v8, ks, vs, g_idx, N, bs)
    err = float(np.abs(out.cpu().numpy() - o_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - o_lse).max())
    announce("  max|out err|", err, "max|lse err|", lerr)
    assert err <= OUT_ATOL and lerr <= 1e-3
    return err


@pytest.mark.parametrize("g", [1, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_decode_groups_and_dims(g, d):
    cfg = synth.scaled(synth.CONFIGS["gqa32k"], name=f"fp8_g{g}d{d}", batch=2, n_kv_heads=2,
                       n_q_heads=2 * g, head_dim=d, seq_len=64 * 150 + 37, top_k=21)
    run_fp8_decode(cfg.name, 61 + g + d, cfg)


def test_fp8_decode_adaptive_lists_and_edges():
    base = synth.CONFIGS["gqa32k"]
    run_fp8_decode("fp8_adaptive", 71, synth.scaled(base, name="fp8_adaptive", batch=2,
                                                    seq_len=64 * 120 + 5), adaptive=True)
    run_fp8_decode("fp8_n1", 72, synth.scaled(base, name="fp8_n1", batch=1, seq_len=1, top_k=3))
    run_fp8_decode("fp8_kall", 73, synth.scaled(base, name="fp8_kall", batch=1, seq_len=64 * 20,
                                                top_k=100))


def test_fp8_decode_full_size_128k():
    cfg = synth.CONFIGS["long128k_15"]
    run_fp8_decode("fp8_long128k_15", synth.DEFAULT_SEED["long128k_15"], cfg)


def test_fp8_longest_supported_cache():
    """The longest FP8 cache a decode call takes at d = 128: 2^25 tokens, so one kv head's
    code rows span exactly 2^32 bytes (addressed by 32-bit byte offsets from the head's
    base).  The GPU quantizes the whole cache; the kept blocks' codes and scales equal the
    oracle's encoding of those blocks bit for bit, the selection (524,285 candidates, the
    strided top-k) equals the oracle's, and the attention over the GPU's codes matches the
    oracle run on the kept blocks gathered into a compact cache (decode attention has no
    positional mask, so only the set of kept tokens matters).  Host work: generating the
    16 GiB of bf16 K and V."""
    import torch
    from parity_rules import check_index_sets
    cfg = synth.scaled(synth.CONFIGS["ctx1m"], name="fp8_ctx32m", batch=1, n_q_heads=8,
                       n_kv_heads=1, seq_len=1 << 25, top_k=64)
    seed, N, bs, d = 18, cfg.seq_len, cfg.block_size, cfg.head_dim
    announce(cfg.name, "seed", seed, "Hq", cfg.n_q_heads, "Hkv 1 d", d, "N", N, "top_k", cfg.top_k)
    t = synth.gen_decode(cfg, seed)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    summ, _ = bsa.build_block_summaries(k, N, bs)
    idx, _ = bsa.select_blocks(q, summ, N, bs, cfg.n_sink, cfg.n_local, cfg.top_k)
    k8, ks = bsa.quantize_kv_fp8(k, N, bs)
    v8, vs = bsa.quantize_kv_fp8(v, N, bs)
    del k, v
    out, lse = bsa.sparse_decode_attn_fp8(q, k8, v8, ks, vs, idx, N, bs)
    torch.cuda.synchronize()
    g_idx = idx.cpu().numpy()
    nb = N // bs
    o_summ = oracle.block_summaries(t["k"], N, bs)
    o_idx, o_scores = oracle.select_blocks(t["q"], o_summ, 1, cfg.n_sink, cfg.n_local,
                                           cfg.top_k, 0.0)
    assert check_index_sets(g_idx, o_idx, o_scores, nb, cfg.n_sink, cfg.n_local) == 0
    blocks = g_idx[0, 0]
    rows = (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
    kc = np.ascontiguousarray(t["k"][:, :, rows])  # the kept blocks, in list order
    vc = np.ascontiguousarray(t["v"][:, :, rows])
    n_c = len(rows)
    ok8, oks = oracle.quantize_fp8(kc, n_c, bs)
    ov8, ovs = oracle.quantize_fp8(vc, n_c, bs)
    g_k8 = k8[:, :, torch.from_numpy(rows).to(k8.device)].cpu().numpy()
    g_v8 = v8[:, :, torch.from_numpy(rows).to(v8.device)].cpu().numpy()
    assert np.array_equal(g_k8, ok8) and np.array_equal(g_v8, ov8), "codes"
    bt = torch.from_numpy(blocks.astype(np.int64)).to(ks.device)
    assert np.array_equal(ks[:, :, bt].cpu().numpy(), oks), "key scales"
    assert np.array_equal(vs[:, :, bt].cpu().numpy(), ovs), "value scales"
    c_idx = np.arange(len(blocks), dtype=np.int32).reshape(1, 1, -1)
    o_out, o_lse = oracle.sparse_decode_attn_fp8(t["q"], ok8, ov8, oks, ovs, c_idx, n_c, bs)
    err = float(np.abs(out.cpu().numpy() - o_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - o_lse).max())
    announce("  max|out err|", err, "max|lse err|", lerr)
    assert err <= OUT_ATOL and lerr <= 1e-3
