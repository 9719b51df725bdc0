"""Seeded synthetic inputs for block-summary sparse attention.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no pooling, scoring, selection or softmax), so the
HIP path and the CPU oracle can both be fed from it without sharing code.

Workloads (sizes follow the decode and chunked-prefill cases this library
is measured on):

* ``tiny``          batch 1, 4 q heads / 4 kv heads, d 64, 1,024 tokens,
                    q/K/V ~ N(0,1); sink 1 + local 2 + top-4 of 13 blocks.
* ``gqa32k``        batch 8, 32/8 heads, d 128, 32,768 tokens, planted
                    power-law block importance; top-74 (~15 % kept).
* ``long128k``      batch 4, 64/8 heads, d 128, 131,072 tokens; top-202
                    (~10 % kept).
* ``long128k_15``   the same shapes at 15 % kept (top-304).
* ``ctx1m``         batch 1, 128/8 heads, d 128, 1,048,576 tokens; top-1635.
* ``prefill256k``   2,048 new queries (tiles of 64) on a 262,144-token cache,
                    32/8 heads, d 128; m=4 top-2048, m=128 dense, window 128.

Planted law (power-law block importance as a stand-in for attention maps
from a trained model): per kv head a unit vector u; per (batch, kv head,
64-token block) a Pareto(alpha=1.5, x_m=1) strength s clipped at 8;
K = N(0,1) + s*u, V = N(0,1), q = N(0,1) + u[kv head of q head].
Every slab draws from its own PCG64 stream keyed by
``[seed, tensor_id, b, kvh]`` so generation order does not matter.
Samples are drawn in fp32 and rounded to bf16 with round-to-nearest-even;
bf16 tensors are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids of the per-slab PRNG streams
_U, _S, _K, _V, _Q = 0, 1, 2, 3, 4
PLANT_BLOCK = 64
PARETO_ALPHA = 1.5
PARETO_CLIP = 8.0


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    block_size: int = 64
    n_sink: int = 1
    n_local: int = 2
    top_k: int = -1
    keep_ratio: float = 0.0
    planted: bool = True


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    prior_len: int        # tokens already in the cache (compressed streams cover these)
    chunk_len: int        # new query tokens, whose K/V are appended after the prior ones
    m_sparse: int = 4
    top_k_sparse: int = 2048
    m_dense: int = 128
    window: int = 128
    q_tile: int = 64
    planted: bool = True


CONFIGS = {
    "tiny": DecodeConfig("tiny", 1, 4, 4, 64, 1024, top_k=4, planted=False),
    "gqa32k": DecodeConfig("gqa32k", 8, 32, 8, 128, 32768, top_k=74),
    "long128k": DecodeConfig("long128k", 4, 64, 8, 128, 131072, top_k=202),
    "long128k_15": DecodeConfig("long128k_15", 4, 64, 8, 128, 131072, top_k=304),
    "ctx1m": DecodeConfig("ctx1m", 1, 128, 8, 128, 1048576, top_k=1635),
    "prefill256k": PrefillConfig("prefill256k", 1, 32, 8, 128, 262144, 2048),
}

DEFAULT_SEED = {"tiny": 1, "gqa32k": 2, "long128k": 3, "long128k_15": 3, "ctx1m": 4,
                "prefill256k": 5}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    return (r >> 16).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 values (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed, tid, b=0, h=0):
    return np.random.default_rng([int(seed), tid, int(b), int(h)])


def _unit_vectors(seed, n_kv_heads, d):
    u = np.empty((n_kv_heads, d), np.float32)
    for h in range(n_kv_heads):
        x = _rng(seed, _U, 0, h).standard_normal(d)
        u[h] = (x / np.linalg.norm(x)).astype(np.float32)
    return u


def _strengths(seed, b, h, n_blocks):
    # Pareto type I, x_m = 1: s = (1-U)^(-1/alpha), clipped at 8
    uni = _rng(seed, _S, b, h).random(n_blocks)
    s = np.power(1.0 - uni, -1.0 / PARETO_ALPHA)
    return np.minimum(s, PARETO_CLIP).astype(np.float32)


def _kv_slab(seed, tid, b, h, n_tok, d, u_h, planted):
    x = _rng(seed, tid, b, h).standard_normal((n_tok, d), dtype=np.float32)
    if planted and tid == _K:
        nblk = -(-n_tok // PLANT_BLOCK)
        s = _strengths(seed, b, h, nblk)
        tok_s = np.repeat(s, PLANT_BLOCK)[:n_tok]
        x += tok_s[:, None] * u_h[None, :]
    return bf16_round(x)


def _gen_kv(seed, batch, n_kv, n_tok, d, u, planted, capacity=None, threads=8):
    cap = n_tok if capacity is None else capacity
    k = np.zeros((batch, n_kv, cap, d), np.uint16)
    v = np.zeros((batch, n_kv, cap, d), np.uint16)
    jobs = [(tid, b, h) for b in range(batch) for h in range(n_kv) for tid in (_K, _V)]

    def work(job):
        tid, b, h = job
        dst = k if tid == _K else v
        dst[b, h, :n_tok] = _kv_slab(seed, tid, b, h, n_tok, d, u[h], planted)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(work, jobs))
    return k, v


def gen_decode(cfg: DecodeConfig, seed: int | None = None, capacity: int | None = None):
    """Returns dict with bf16 (uint16) q [B][Hq][d], k, v [B][Hkv][capacity][d].

    Tokens past ``seq_len`` (when capacity > seq_len) are zero.
    """
    seed = DEFAULT_SEED.get(cfg.name, 0) if seed is None else seed
    g = cfg.n_q_heads // cfg.n_kv_heads
    d = cfg.head_dim
    u = _unit_vectors(seed, cfg.n_kv_heads, d)
    if not cfg.planted:
        u = np.zeros_like(u)
    k, v = _gen_kv(seed, cfg.batch, cfg.n_kv_heads, cfg.seq_len, d, u, cfg.planted, capacity)
    q = np.empty((cfg.batch, cfg.n_q_heads, d), np.uint16)
    for b in range(cfg.batch):
        x = _rng(seed, _Q, b, 0).standard_normal((cfg.n_q_heads, d), dtype=np.float32)
        x += np.repeat(u, g, axis=0)
        q[b] = bf16_round(x)
    return {"q": q, "k": k, "v": v}


def gen_prefill(cfg: PrefillConfig, seed: int | None = None):
    """Returns dict with bf16 q [B][C][Hq][d], k, v [B][Hkv][P+C][d]."""
    seed = DEFAULT_SEED.get(cfg.name, 0) if seed is None else seed
    g = cfg.n_q_heads // cfg.n_kv_heads
    d = cfg.head_dim
    u = _unit_vectors(seed, cfg.n_kv_heads, d)
    if not cfg.planted:
        u = np.zeros_like(u)
    n_tok = cfg.prior_len + cfg.chunk_len
    k, v = _gen_kv(seed, cfg.batch, cfg.n_kv_heads, n_tok, d, u, cfg.planted)
    q = np.empty((cfg.batch, cfg.chunk_len, cfg.n_q_heads, d), np.uint16)
    for b in range(cfg.batch):
        x = _rng(seed, _Q, b, 0).standard_normal((cfg.chunk_len, cfg.n_q_heads, d),
                                                 dtype=np.float32)
        x += np.repeat(u, g, axis=0)[None, :, :]
        q[b] = bf16_round(x)
    return {"q": q, "k": k, "v": v}


def scaled(cfg, **kw):
    """A copy of a config with some sizes replaced (for parity at reduced size)."""
    return dataclasses.replace(cfg, **kw)
