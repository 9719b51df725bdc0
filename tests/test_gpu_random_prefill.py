"""Randomised GPU parity of the chunked prefill against the oracle.

20 seeded cases draw the batch, kv heads, group size (64-query tiles of 64, 128
or 256 (query, head) rows), prior length (log-uniform from 64 to 300,000 tokens),
chunk length, both pooling ratios, top-k, window, the combine mode and optional
sink logits (every third case selects with the fp32-means indexer, the others
with the bf16 compressed keys); each case checks the tile selections (near-tie rule) and the
outputs and per-branch lse against the oracle evaluated on the GPU's selection,
as the fixed-shape tests do (every row for chunks up to 128 queries, 40 sampled
rows beyond).  8 more cases draw longer chunks in tiles of 16-64 queries (up to 57
tiles).  Every case prints its parameters before any GPU call.
"""
import math

import numpy as np
import pytest

import long_context_block_summary_amd as bsa
from long_context_block_summary_amd import synth
from test_gpu_prefill import run_prefill_case

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
    rng = np.random.default_rng(9000 + i)
    hkv, g = int(rng.choice([1, 2])), int(rng.choice([1, 2, 4]))
    C = int(rng.integers(1, 261))
    cfg = synth.PrefillConfig(
        name=f"pf_rand{i}", batch=int(rng.integers(1, 3)), n_q_heads=hkv * g, n_kv_heads=hkv,
        head_dim=128, prior_len=int(math.exp(rng.uniform(math.log(64), math.log(300000)))),
        chunk_len=C,
        m_sparse=int(rng.choice([2, 4, 8])), top_k_sparse=int(rng.integers(1, 701)),
        m_dense=int(rng.choice([16, 64, 128, 256])), window=int(rng.integers(1, 401)),
        planted=bool(rng.integers(0, 2)))
    combine = int(rng.integers(0, 2))
    sink = rng.uniform(-3.0, 3.0, hkv * g).astype(np.float32) if rng.integers(0, 2) else None
    rows = None if C <= 128 else np.sort(rng.choice(C, 40, replace=False)).tolist()
    return cfg, int(rng.integers(0, 10**6)), combine, sink, rows


@pytest.mark.parametrize("i", range(20))
def test_random_prefill_shapes(i):
    cfg, seed, combine, sink, rows = draw_case(i)
    indexer = bsa.INDEXER_F32 if i % 3 == 2 else bsa.INDEXER_BF16
    run_prefill_case(cfg, seed, rows=rows, combine=combine, sink=sink, indexer=indexer)


@pytest.mark.parametrize("i", range(8))
def test_random_prefill_many_tiles(i):
    """Seeded random prefill with longer chunks (100-900 queries) in tiles of 16, 32 or 64
    queries (up to 57 tiles: three or four blocks of 16 tiles in the scores kernels), priors
    of 1,000-120,000 tokens, top-k up to 3,000, either indexer and combine mode; 24 sampled
    rows."""
    rng = np.random.default_rng(78000 + i)
    hkv, g = int(rng.choice([1, 2])), int(rng.choice([1, 2, 4]))
    qt = int(rng.choice([16, 32, 64]))
    while qt * g not in (64, 128, 256):
        qt *= 2
    C = int(rng.integers(100, 900))
    cfg = synth.PrefillConfig(
        name=f"pf_tiles_rand{i}", batch=1, n_q_heads=hkv * g, n_kv_heads=hkv, head_dim=128,
        prior_len=int(rng.integers(1000, 120000)), chunk_len=C, q_tile=qt,
        m_sparse=int(rng.choice([4, 8])), top_k_sparse=int(rng.integers(1, 3000)),
        m_dense=int(rng.choice([64, 128])), window=int(rng.integers(1, 300)),
        planted=bool(rng.integers(0, 2)))
    rows = np.sort(rng.choice(C, 24, replace=False)).tolist()
    run_prefill_case(cfg, int(rng.integers(0, 10**6)), rows=rows,
                     combine=int(rng.integers(0, 2)), indexer=int(rng.integers(0, 2)))
