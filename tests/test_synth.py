"""Seeded input generators (long_context_block_summary_amd.synth): the same seed gives the same
tensors whatever the generation order or thread count, slabs are keyed by (seed, tensor,
batch, kv head), and the planted block strengths follow the stated Pareto law."""
import numpy as np

from long_context_block_summary_amd import synth


def _small(**kw):
    base = dict(name="t0", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64, seq_len=64 * 20 + 5,
                top_k=4)
    base.update(kw)
    return synth.DecodeConfig(**base)


def test_same_seed_same_tensors_any_thread_count():
    cfg = _small()
    a = synth.gen_decode(cfg, 11)
    b = synth.gen_decode(cfg, 11)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key]), key
    u = synth._unit_vectors(11, cfg.n_kv_heads, cfg.head_dim)
    k1, v1 = synth._gen_kv(11, cfg.batch, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim, u, True,
                           threads=1)
    assert np.array_equal(k1, a["k"]) and np.array_equal(v1, a["v"])
    c = synth.gen_decode(cfg, 12)
    assert not np.array_equal(a["k"], c["k"]) and not np.array_equal(a["q"], c["q"])


def test_slabs_keyed_by_batch_and_head():
    """A (batch, kv head) slab does not depend on how many others are generated with it."""
    a = synth.gen_decode(_small(batch=2), 5)
    b = synth.gen_decode(_small(batch=3), 5)
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key][:2]), key
    # capacity beyond seq_len: the extra rows are zero, the rest unchanged
    cfg = _small()
    c = synth.gen_decode(cfg, 5, capacity=cfg.seq_len + 100)
    assert np.array_equal(c["k"][:, :, :cfg.seq_len], a["k"])
    assert not c["k"][:, :, cfg.seq_len:].any() and not c["v"][:, :, cfg.seq_len:].any()


def test_pareto_strengths_and_clip_fraction():
    """s = (1 - U)^(-1/1.5) >= 1, clipped at 8: P(s = 8) = 8^-1.5 (about 0.0442)."""
    n = 200_000
    s = synth._strengths(3, 0, 0, n).astype(np.float64)
    assert s.min() >= 1.0 and s.max() == synth.PARETO_CLIP
    p = synth.PARETO_CLIP ** -synth.PARETO_ALPHA
    frac = np.mean(s == synth.PARETO_CLIP)
    assert abs(frac - p) < 5 * np.sqrt(p * (1 - p) / n), (frac, p)
    # median of the Pareto law: 2^(1/alpha)
    assert abs(np.median(s) - 2 ** (1 / synth.PARETO_ALPHA)) < 0.02


def test_planted_blocks_follow_their_strengths():
    """K = N(0,1) + s u per 64-token block: the block means projected on u track s."""
    cfg = _small(batch=1, n_kv_heads=1, n_q_heads=4, head_dim=128, seq_len=64 * 400)
    t = synth.gen_decode(cfg, 7)
    u = synth._unit_vectors(7, 1, 128)[0].astype(np.float64)
    k = synth.bf16_to_f32(t["k"][0, 0]).astype(np.float64).reshape(400, 64, 128)
    proj = k.mean(axis=1) @ u
    s = synth._strengths(7, 0, 0, 400).astype(np.float64)
    assert np.corrcoef(proj, s)[0, 1] > 0.95
    # and the unplanted tiny config has no planted direction
    tiny = synth.gen_decode(synth.CONFIGS["tiny"])
    kt = synth.bf16_to_f32(tiny["k"]).astype(np.float64)
    assert abs(kt.mean()) < 0.05 and abs(kt.std() - 1.0) < 0.05
