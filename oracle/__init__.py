"""ctypes wrapper of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
loads it and shares no code with it.

All wrappers take numpy arrays: bf16 tensors as uint16 bit patterns, results
as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("BSA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared"]


def build(extra_flags=(), out=LIB_PATH):
    """Compile oracle.c with gcc (plain C99, fp64, no fast-math)."""
    cmd = ["gcc", *_CFLAGS, *extra_flags, os.path.join(_HERE, "oracle.c"), "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path=LIB_PATH):
    global _lib
    if path == LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    i32, f64, vp = ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    lib.oracle_num_blocks.argtypes = [i32, i32]
    lib.oracle_num_blocks.restype = i32
    lib.oracle_num_kept.argtypes = [i32, i32, i32, i32, f64]
    lib.oracle_num_kept.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = None
    lib.oracle_round_bf16.argtypes = [f64]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_block_summaries.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp]
    lib.oracle_block_summaries.restype = ctypes.c_int
    lib.oracle_block_summaries_f32.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp]
    lib.oracle_block_summaries_f32.restype = ctypes.c_int
    lib.oracle_select_blocks.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f64,
                                         vp, vp]
    lib.oracle_select_blocks.restype = ctypes.c_int
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = f64
    lib.oracle_e4m3_encode.argtypes = [f64]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_quantize_fp8.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.oracle_quantize_fp8.restype = ctypes.c_int
    lib.oracle_sparse_decode_attn_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                  i32, i32, i32, i32, i32, f64, vp, vp]
    lib.oracle_sparse_decode_attn_fp8.restype = ctypes.c_int
    lib.oracle_adaptive_bounds.argtypes = [i32, i32, i32, f64, f64, vp, vp]
    lib.oracle_adaptive_bounds.restype = ctypes.c_int32
    lib.oracle_select_blocks_adaptive.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                                  f64, f64, f64, vp, vp, vp]
    lib.oracle_select_blocks_adaptive.restype = ctypes.c_int
    lib.oracle_sparse_decode_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                              i32, f64, vp, vp, vp]
    lib.oracle_sparse_decode_attn.restype = ctypes.c_int
    lib.oracle_sparse_prefill_attn.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                               i32, i32, i32, i32, i32, f64, vp, vp, i32, i32, i32,
                                               vp, vp, vp, vp, vp, vp]
    lib.oracle_sparse_prefill_attn.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def num_blocks(n, m, lib=None):
    return (lib or load()).oracle_num_blocks(n, m)


def num_kept(nb, n_sink, n_local, top_k, keep_ratio=0.0, lib=None):
    return (lib or load()).oracle_num_kept(nb, n_sink, n_local, top_k, float(keep_ratio))


def num_threads(lib=None):
    return (lib or load()).oracle_num_threads()


def set_threads(n, lib=None):
    (lib or load()).oracle_set_threads(int(n))


def round_bf16(x, lib=None):
    return (lib or load()).oracle_round_bf16(float(x))


def block_summaries(x, seq_len, block_size, lib=None):
    """x: uint16 [B][H][stride][d] -> float64 [B][H][nb][d]."""
    lib = lib or load()
    x = _u16(x)
    B, H, stride, d = x.shape
    nb = -(-seq_len // block_size)
    out = np.empty((B, H, nb, d), np.float64)
    rc = lib.oracle_block_summaries(_p(x), B, H, seq_len, stride, d, block_size, _p(out))
    if rc:
        raise ValueError(f"oracle_block_summaries rc={rc}")
    return out


def block_summaries_f32(x, seq_len, block_size, lib=None):
    """x: uint16 [B][H][stride][d] -> float32 [B][H][nb][d]: the fp32 running sum in token
    order, then one fp32 division by the block's token count."""
    lib = lib or load()
    x = _u16(x)
    B, H, stride, d = x.shape
    nb = -(-seq_len // block_size)
    out = np.empty((B, H, nb, d), np.float32)
    rc = lib.oracle_block_summaries_f32(_p(x), B, H, seq_len, stride, d, block_size, _p(out))
    if rc:
        raise ValueError(f"oracle_block_summaries_f32 rc={rc}")
    return out


def select_blocks(q, summaries, n_kv_heads, n_sink=1, n_local=2, top_k=-1, keep_ratio=0.0,
                  lib=None):
    """q: uint16 [B][Hq][d]; summaries float64 [B][Hkv][nb][d].

    Returns (idx int32 [B][Hkv][n_keep] ascending, scores float64 [B][Hkv][nb]
    with NaN outside the candidate range)."""
    lib = lib or load()
    q = _u16(q)
    summaries = np.ascontiguousarray(summaries, dtype=np.float64)
    B, Hq, d = q.shape
    nb = summaries.shape[2]
    n_keep = lib.oracle_num_kept(nb, n_sink, n_local, top_k, float(keep_ratio))
    idx = np.empty((B, n_kv_heads, n_keep), np.int32)
    scores = np.empty((B, n_kv_heads, nb), np.float64)
    rc = lib.oracle_select_blocks(_p(q), _p(summaries), B, Hq, n_kv_heads, d, nb, n_sink,
                                  n_local, top_k, float(keep_ratio), _p(idx), _p(scores))
    if rc:
        raise ValueError(f"oracle_select_blocks rc={rc}")
    return idx, scores


def e4m3_value(code, lib=None):
    return (lib or load()).oracle_e4m3_value(int(code))


def e4m3_encode(y, lib=None):
    return int((lib or load()).oracle_e4m3_encode(float(y)))


def quantize_fp8(x, seq_len, block_size=64, sstride=0, lib=None):
    """x uint16 (bf16 bits) [B][H][stride][d] -> (codes uint8 [B][H][stride][d], rows >= seq_len
    zero; scales float32 [B][H][S], S = sstride or ceil(seq_len / block_size))."""
    lib = lib or load()
    x = _u16(x)
    B, H, stride, d = x.shape
    S = sstride or -(-seq_len // block_size)
    out = np.zeros((B, H, stride, d), np.uint8)
    sc = np.zeros((B, H, S), np.float32)
    rc = lib.oracle_quantize_fp8(_p(x), B, H, seq_len, stride, d, block_size, S, _p(out), _p(sc))
    if rc:
        raise ValueError(f"oracle_quantize_fp8 rc={rc}")
    return out, sc


def sparse_decode_attn_fp8(q, k8, v8, kscales, vscales, idx, seq_len, block_size=64, scale=0.0,
                           lib=None):
    """Attention over the dequantized FP8 cache; returns (out [B][Hq][d], lse [B][Hq])."""
    lib = lib or load()
    q = _u16(q)
    k8 = np.ascontiguousarray(k8, dtype=np.uint8)
    v8 = np.ascontiguousarray(v8, dtype=np.uint8)
    kscales = np.ascontiguousarray(kscales, dtype=np.float32)
    vscales = np.ascontiguousarray(vscales, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, Hq, d = q.shape
    Hkv, stride = k8.shape[1], k8.shape[2]
    out = np.empty((B, Hq, d), np.float64)
    lse = np.empty((B, Hq), np.float64)
    rc = lib.oracle_sparse_decode_attn_fp8(_p(q), _p(k8), _p(v8), _p(kscales), _p(vscales),
                                           _p(idx), idx.shape[2], B, Hq, Hkv, d, seq_len, stride,
                                           block_size, kscales.shape[2], float(scale), _p(out),
                                           _p(lse))
    if rc:
        raise ValueError(f"oracle_sparse_decode_attn_fp8 rc={rc}")
    return out, lse


def adaptive_bounds(nb, n_sink, n_local, ratio_min, ratio_max, lib=None):
    """(width of the kept lists, k_lo, k_hi) of an anchor-adaptive selection."""
    lib = lib or load()
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    w = lib.oracle_adaptive_bounds(nb, n_sink, n_local, float(ratio_min), float(ratio_max),
                                   ctypes.byref(lo), ctypes.byref(hi))
    if w < 0:
        raise ValueError("invalid adaptive selection bounds")
    return w, lo.value, hi.value


def select_blocks_adaptive(q, summaries, n_kv_heads, n_sink=1, n_local=2, ratio_min=0.1,
                           ratio_max=0.2, margin=0.0, lib=None):
    """Anchor-adaptive selection.  Returns (idx int32 [B][Hkv][width] ascending and padded
    with -1, count int32 [B][Hkv] kept blocks, scores float64 [B][Hkv][nb] of every block)."""
    lib = lib or load()
    q = _u16(q)
    summaries = np.ascontiguousarray(summaries, dtype=np.float64)
    B, Hq, d = q.shape
    nb = summaries.shape[2]
    width, _, _ = adaptive_bounds(nb, n_sink, n_local, ratio_min, ratio_max, lib)
    idx = np.empty((B, n_kv_heads, width), np.int32)
    cnt = np.empty((B, n_kv_heads), np.int32)
    scores = np.empty((B, n_kv_heads, nb), np.float64)
    rc = lib.oracle_select_blocks_adaptive(_p(q), _p(summaries), B, Hq, n_kv_heads, d, nb,
                                           n_sink, n_local, float(ratio_min), float(ratio_max),
                                           float(margin), _p(idx), _p(cnt), _p(scores))
    if rc:
        raise ValueError(f"oracle_select_blocks_adaptive rc={rc}")
    return idx, cnt, scores


def sparse_decode_attn(q, k, v, idx, seq_len, block_size=64, scale=0.0, want_weights=False,
                       lib=None):
    """q uint16 [B][Hq][d]; k, v uint16 [B][Hkv][stride][d]; idx int32 [B][Hkv][n_keep].

    Returns (out [B][Hq][d], lse [B][Hq], weights [B][Hq][n_keep*bs] or None)."""
    lib = lib or load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, Hq, d = q.shape
    Hkv, stride = k.shape[1], k.shape[2]
    n_keep = idx.shape[2]
    out = np.empty((B, Hq, d), np.float64)
    lse = np.empty((B, Hq), np.float64)
    w = np.empty((B, Hq, n_keep * block_size), np.float64) if want_weights else None
    rc = lib.oracle_sparse_decode_attn(_p(q), _p(k), _p(v), _p(idx), n_keep, B, Hq, Hkv, d,
                                       seq_len, stride, block_size, float(scale), _p(out),
                                       _p(lse), _p(w))
    if rc:
        raise ValueError(f"oracle_sparse_decode_attn rc={rc}")
    return out, lse, w


def sparse_prefill_attn(q, k, v, prior_len, m_sparse=4, top_k=2048, m_dense=128, window=128,
                        q_tile=64, scale=0.0, sel_in=None, rows=None, want_branches=False,
                        want_sel=False, want_sel_scores=False, combine=0, sink_logits=None,
                        indexer=0, lib=None):
    """q uint16 [B][C][Hq][d]; k, v uint16 [B][Hkv][stride][d] (prior + chunk tokens).
    combine 0 averages the three branches, 1 takes one softmax over their
    concatenated logits; sink_logits [Hq] (natural log) or None.  indexer 0 scores the
    tiles' pooled queries against the bf16 compressed keys (the bf16 rounding of the fp32
    token-order means), 1 against the exact means.

    Returns dict: out [B][R][Hq][d], lse3 [3][B][R][Hq], and optionally
    branches [3][B][R][Hq][d], sel [B][tiles][Hkv][k'], sel_scores."""
    lib = lib or load()
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, C, Hq, d = q.shape
    Hkv, stride = k.shape[1], k.shape[2]
    E4 = -(-prior_len // m_sparse)
    kk = min(top_k, E4)
    n_tiles = -(-C // q_tile)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int32)
    R = C if rows is None else len(rows)
    out = np.empty((B, R, Hq, d), np.float64)
    lse3 = np.empty((3, B, R, Hq), np.float64)
    br = np.empty((3, B, R, Hq, d), np.float64) if want_branches else None
    sel = np.empty((B, n_tiles, Hkv, kk), np.int32) if want_sel else None
    ss = np.empty((B, n_tiles, Hkv, E4), np.float64) if want_sel_scores else None
    if sel_in is not None:
        sel_in = np.ascontiguousarray(sel_in, dtype=np.int32)
        assert sel_in.shape == (B, n_tiles, Hkv, kk)
    if sink_logits is not None:
        sink_logits = np.ascontiguousarray(sink_logits, dtype=np.float64)
        assert sink_logits.shape == (Hq,)
    rc = lib.oracle_sparse_prefill_attn(_p(q), C, _p(k), _p(v), B, prior_len, Hq, Hkv, d,
                                        stride, m_sparse, top_k, m_dense, window, q_tile,
                                        float(scale), _p(sel_in), _p(rows), R, int(combine),
                                        int(indexer), _p(sink_logits), _p(out), _p(br), _p(lse3), _p(sel),
                                        _p(ss))
    if rc:
        raise ValueError(f"oracle_sparse_prefill_attn rc={rc}")
    return {"out": out, "lse3": lse3, "branches": br, "sel": sel, "sel_scores": ss}
