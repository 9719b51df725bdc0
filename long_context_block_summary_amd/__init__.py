"""Block-summary sparse attention for MI355X (gfx950).

Thin ctypes binding of libbsa.so: argument marshalling only.  Every step of
the path runs in the library's HIP kernels; torch provides device memory and
the current stream.  The functions carry the names of the C entry points in
include/bsa.h.  There is no CPU fallback: if libbsa.so is missing or a call
fails, a BsaError is raised.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libbsa.so")

BSA_OK, BSA_INVALID_ARG, BSA_UNSUPPORTED, BSA_WORKSPACE_TOO_SMALL, BSA_HIP_ERROR = 0, -1, -2, -3, -4
SIZE_MAX = ctypes.c_size_t(-1).value


class BsaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class bsa_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("seq_stride", ctypes.c_int32),
                ("summary_stride", ctypes.c_int32)]


class bsa_select_cfg(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("n_sink_blocks", ctypes.c_int32),
                ("n_local_blocks", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("keep_ratio", ctypes.c_double), ("adaptive", ctypes.c_int32),
                ("keep_ratio_max", ctypes.c_double), ("anchor_margin", ctypes.c_double),
                ("summaries_bf16", ctypes.c_int32)]


class bsa_prefill_cfg(ctypes.Structure):
    _fields_ = [("m_sparse", ctypes.c_int32), ("top_k_sparse", ctypes.c_int32),
                ("m_dense", ctypes.c_int32), ("window", ctypes.c_int32),
                ("q_tile", ctypes.c_int32), ("combine", ctypes.c_int32),
                ("indexer", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libbsa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    i32, f32, vp, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    L.bsa_num_blocks.argtypes, L.bsa_num_blocks.restype = [i32, i32], i32
    L.bsa_num_kept.argtypes, L.bsa_num_kept.restype = [i32, P(bsa_select_cfg)], i32
    L.bsa_select_workspace_size.argtypes = [P(bsa_shape), P(bsa_select_cfg)]
    L.bsa_select_workspace_size.restype = sz
    L.bsa_decode_workspace_size.argtypes = [P(bsa_shape), i32, i32, i32]
    L.bsa_decode_workspace_size.restype = sz
    L.bsa_decode_step_workspace_size.argtypes = [P(bsa_shape), P(bsa_select_cfg)]
    L.bsa_decode_step_workspace_size.restype = sz
    L.bsa_prefill_workspace_size.argtypes = [P(bsa_shape), i32, P(bsa_prefill_cfg)]
    L.bsa_prefill_workspace_size.restype = sz
    L.bsa_status_string.argtypes, L.bsa_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    L.build_block_summaries.argtypes = [vp, P(bsa_shape), i32, vp, vp, vp]
    L.update_block_summaries.argtypes = [vp, P(bsa_shape), i32, i32, vp, vp, vp]
    L.append_kv.argtypes = [vp, vp, vp, vp, P(bsa_shape), i32, i32, vp, vp, vp]
    L.select_blocks.argtypes = [vp, vp, P(bsa_shape), P(bsa_select_cfg), vp, vp, vp, sz, vp]
    L.sparse_decode_attn.argtypes = [vp, vp, vp, vp, i32, P(bsa_shape), i32, f32, vp, vp, vp, sz,
                                     vp]
    L.sparse_decode_attn_split.argtypes = [vp, vp, vp, vp, i32, P(bsa_shape), i32, f32, vp, vp,
                                           vp, sz, i32, vp]
    L.sparse_decode_partials.argtypes = [vp, vp, vp, vp, i32, P(bsa_shape), i32, f32, vp, sz, i32,
                                         vp]
    L.sparse_decode_merge.argtypes = [P(bsa_shape), i32, i32, i32, vp, sz, vp, vp, vp]
    L.sparse_decode_step.argtypes = [vp, vp, vp, vp, P(bsa_shape), P(bsa_select_cfg), vp, f32, vp,
                                     vp, vp, sz, vp]
    L.sparse_prefill_attn.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, P(bsa_shape),
                                      P(bsa_prefill_cfg), f32, vp, vp, vp, vp, vp, sz, vp]
    L.select_prefill_entries.argtypes = [vp, i32, vp, vp, P(bsa_shape), P(bsa_prefill_cfg), vp,
                                         vp, sz, vp]
    L.sparse_prefill_attn_selected.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                               P(bsa_shape), P(bsa_prefill_cfg), f32, vp, vp, vp,
                                               vp]
    L.quantize_kv_fp8.argtypes = [vp, P(bsa_shape), i32, vp, vp, vp]
    L.sparse_decode_attn_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, P(bsa_shape), i32, f32, vp,
                                         vp, vp, sz, vp]
    for fn in ("quantize_kv_fp8", "sparse_decode_attn_fp8",
               "build_block_summaries", "update_block_summaries", "append_kv",
               "select_blocks", "sparse_decode_attn",
               "sparse_decode_attn_split", "sparse_decode_partials", "sparse_decode_merge",
               "sparse_prefill_attn", "select_prefill_entries",
               "sparse_prefill_attn_selected", "sparse_decode_step"):
        getattr(L, fn).restype = ctypes.c_int
    _lib = L
    return L


def _check(fn, status):
    if status != BSA_OK:
        raise BsaError(fn, status, lib().bsa_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dtype, ndim):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {ndim}-d {dtype} tensor, got "
                        f"{t.dtype} {tuple(t.shape)}")


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, seq_len, seq_stride, summary_stride=0):
    return bsa_shape(batch, n_q_heads, n_kv_heads, head_dim, seq_len, seq_stride, summary_stride)


def select_cfg(block_size=64, n_sink=1, n_local=2, top_k=-1, keep_ratio=0.0, adaptive=False,
               keep_ratio_max=0.0, anchor_margin=0.0, summaries_bf16=False):
    """Selection parameters; adaptive=True keeps between keep_ratio and keep_ratio_max of the
    blocks per (b, kv head), set by the anchors' scores (lists padded with -1);
    summaries_bf16 when the summaries are bf16 rather than fp32."""
    return bsa_select_cfg(block_size, n_sink, n_local, top_k, keep_ratio, int(adaptive),
                          keep_ratio_max, anchor_margin, int(summaries_bf16))


def _summaries_bf16(summaries):
    """True for bf16 summaries, False for fp32 ones (a contiguous 4-d device tensor)."""
    import torch
    if isinstance(summaries, torch.Tensor) and summaries.dtype == torch.bfloat16:
        _need(summaries, "summaries", torch.bfloat16, 4)
        return True
    _need(summaries, "summaries", torch.float32, 4)
    return False


COMBINE_AVERAGE, COMBINE_CONCAT = 0, 1
INDEXER_BF16, INDEXER_F32 = 0, 1


def prefill_cfg(m_sparse=4, top_k_sparse=2048, m_dense=128, window=128, q_tile=64,
                combine=COMBINE_AVERAGE, indexer=INDEXER_BF16):
    """Prefill parameters; indexer picks the keys the branch-A selection scores against:
    INDEXER_BF16 the bf16 compressed keys (the entries branch A attends), INDEXER_F32 the
    fp32 means."""
    return bsa_prefill_cfg(m_sparse, top_k_sparse, m_dense, window, q_tile, combine, indexer)


def num_blocks(n, m):
    return lib().bsa_num_blocks(n, m)


def num_kept(nb, cfg):
    return lib().bsa_num_kept(nb, ctypes.byref(cfg))


# ------------------------------------------------------------------ entry points

def build_block_summaries(x, seq_len, block_size, want_f32=True, want_bf16=False,
                          out_f32=None, out_bf16=None, summary_stride=0):
    """x bf16 [B][H][stride][d] -> (fp32 [B][H][S][d] or None, bf16 [B][H][S][d] or None),
    S = summary_stride or nb = ceil(seq_len / block_size) when that is 0."""
    import torch
    _need(x, "x", torch.bfloat16, 4)
    B, H, stride, d = x.shape
    S = summary_stride or num_blocks(seq_len, block_size)
    if want_f32 and out_f32 is None:
        out_f32 = torch.empty((B, H, S, d), dtype=torch.float32, device=x.device)
    if want_bf16 and out_bf16 is None:
        out_bf16 = torch.empty((B, H, S, d), dtype=torch.bfloat16, device=x.device)
    shape = make_shape(B, H, H, d, seq_len, stride, summary_stride)
    _check("build_block_summaries",
           lib().build_block_summaries(_ptr(x), ctypes.byref(shape), block_size, _ptr(out_f32),
                                       _ptr(out_bf16), _stream(x.device)))
    return out_f32, out_bf16


def update_block_summaries(x, seq_len, block_size, first_token, out_f32=None, out_bf16=None):
    """Recompute, in place, the summaries of the blocks holding tokens [first_token, seq_len)
    of x bf16 [B][H][stride][d]; out_* [B][H][S][d] as from build_block_summaries."""
    import torch
    _need(x, "x", torch.bfloat16, 4)
    B, H, stride, d = x.shape
    ref = out_f32 if out_f32 is not None else out_bf16
    if ref is None:
        raise ValueError("an output buffer is required")
    shape = make_shape(B, H, H, d, seq_len, stride, ref.shape[2])
    _check("update_block_summaries",
           lib().update_block_summaries(_ptr(x), ctypes.byref(shape), block_size, first_token,
                                        _ptr(out_f32), _ptr(out_bf16), _stream(x.device)))
    return out_f32, out_bf16


def append_kv(k_new, v_new, k_cache, v_cache, seq_len, block_size=64, summaries=None):
    """Write k_new, v_new bf16 [B][Hkv][n][d] into the caches at [seq_len, seq_len + n); with
    `summaries` (fp32 or bf16 [B][Hkv][S][d]) also refresh the summaries of the blocks they
    land in."""
    import torch
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache),
                    ("v_cache", v_cache)):
        _need(t, name, torch.bfloat16, 4)
    B, H, n, d = k_new.shape
    if tuple(v_new.shape) != (B, H, n, d) or k_cache.shape[:2] != (B, H) or \
            tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[3] != d:
        raise ValueError("append_kv: shapes do not match")
    S, s32, s16 = 0, None, None
    if summaries is not None:
        if _summaries_bf16(summaries):
            s16 = summaries
        else:
            s32 = summaries
        S = summaries.shape[2]
    shape = make_shape(B, H, H, d, seq_len, k_cache.shape[2], S)
    _check("append_kv", lib().append_kv(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                        ctypes.byref(shape), n, block_size, _ptr(s32), _ptr(s16),
                                        _stream(k_new.device)))


def select_blocks(q, summaries, seq_len, block_size=64, n_sink=1, n_local=2, top_k=-1,
                  keep_ratio=0.0, want_scores=False, block_idx=None, workspace=None,
                  adaptive=False, keep_ratio_max=0.0, anchor_margin=0.0):
    """q bf16 [B][Hq][d], summaries fp32 or bf16 [B][Hkv][nb][d] -> (idx int32
    [B][Hkv][n_keep], scores)."""
    import torch
    _need(q, "q", torch.bfloat16, 3)
    sb = _summaries_bf16(summaries)
    B, Hq, d = q.shape
    Hkv, S = summaries.shape[1], summaries.shape[2]
    nb = num_blocks(seq_len, block_size)
    if S < nb:
        raise ValueError(f"summaries hold {S} blocks, {nb} are in use")
    cfg = select_cfg(block_size, n_sink, n_local, top_k, keep_ratio, adaptive, keep_ratio_max,
                     anchor_margin, summaries_bf16=sb)
    n_keep = num_kept(nb, cfg)
    if n_keep < 0:
        raise ValueError("invalid selection config")
    shape = make_shape(B, Hq, Hkv, d, seq_len, seq_len, S)
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, n_keep), dtype=torch.int32, device=q.device)
    scores = None
    if want_scores:
        scores = torch.full((B, Hkv, nb), float("nan"), dtype=torch.float32, device=q.device)
    ws_bytes = lib().bsa_select_workspace_size(ctypes.byref(shape), ctypes.byref(cfg))
    if ws_bytes == SIZE_MAX:
        raise ValueError("invalid select arguments")
    if workspace is None and scores is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check("select_blocks",
           lib().select_blocks(_ptr(q), _ptr(summaries), ctypes.byref(shape), ctypes.byref(cfg),
                               _ptr(block_idx), _ptr(scores), _ptr(workspace),
                               workspace.numel() if workspace is not None else 0,
                               _stream(q.device)))
    return block_idx, scores


def sparse_decode_step(q, k, v, summaries, seq_len, block_size=64, n_sink=1, n_local=2, top_k=-1,
                       keep_ratio=0.0, scale=0.0, block_idx=None, out=None, lse=None,
                       workspace=None, want_lse=True):
    """select_blocks then sparse_decode_attn in one call (the selection fused into the
    attention launch where it fits).  Returns (out, lse or None, block_idx)."""
    import torch
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    sb = _summaries_bf16(summaries)
    B, Hq, d = q.shape
    Hkv, stride = k.shape[1], k.shape[2]
    S = summaries.shape[2]
    if tuple(v.shape) != tuple(k.shape) or summaries.shape[:2] != (B, Hkv):
        raise ValueError("k, v and summaries shapes disagree")
    nb = num_blocks(seq_len, block_size)
    if S < nb:
        raise ValueError(f"summaries hold {S} blocks, {nb} are in use")
    cfg = select_cfg(block_size, n_sink, n_local, top_k, keep_ratio, summaries_bf16=sb)
    n_keep = num_kept(nb, cfg)
    if n_keep < 1:
        raise ValueError("invalid selection config")
    shape = make_shape(B, Hq, Hkv, d, seq_len, stride, S)
    ws_bytes = lib().bsa_decode_step_workspace_size(ctypes.byref(shape), ctypes.byref(cfg))
    if ws_bytes == SIZE_MAX:
        raise ValueError("invalid decode step arguments")
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if block_idx is None:
        block_idx = torch.empty((B, Hkv, n_keep), dtype=torch.int32, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check("sparse_decode_step",
           lib().sparse_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(summaries),
                                    ctypes.byref(shape), ctypes.byref(cfg), _ptr(block_idx), scale,
                                    _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                    _stream(q.device)))
    return out, lse, block_idx


def decode_step_workspace_size(B, Hq, Hkv, d, seq_len, block_size=64, n_sink=1, n_local=2,
                               top_k=-1, keep_ratio=0.0, summaries_bf16=False):
    """Bytes of workspace sparse_decode_step needs (block scores, then split partials)."""
    shape = make_shape(B, Hq, Hkv, d, seq_len, seq_len)
    cfg = select_cfg(block_size, n_sink, n_local, top_k, keep_ratio, summaries_bf16=summaries_bf16)
    n = lib().bsa_decode_step_workspace_size(ctypes.byref(shape), ctypes.byref(cfg))
    if n == SIZE_MAX:
        raise ValueError("invalid decode step arguments")
    return max(int(n), 16)


def decode_workspace_size(B, Hq, Hkv, d, seq_len, n_keep, block_size=64, n_splits=0):
    shape = make_shape(B, Hq, Hkv, d, seq_len, seq_len)
    return lib().bsa_decode_workspace_size(ctypes.byref(shape), n_keep, block_size, n_splits)


def sparse_decode_attn(q, k, v, block_idx, seq_len, block_size=64, scale=0.0, n_splits=0,
                       out=None, lse=None, workspace=None, want_lse=True):
    """q bf16 [B][Hq][d]; k, v bf16 [B][Hkv][stride][d]; block_idx int32 [B][Hkv][n_keep].

    Returns (out fp32 [B][Hq][d], lse fp32 [B][Hq] or None)."""
    import torch
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(block_idx, "block_idx", torch.int32, 3)
    B, Hq, d = q.shape
    Hkv, stride = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or block_idx.shape[:2] != (B, Hkv):
        raise ValueError("k, v and block_idx shapes disagree")
    n_keep = block_idx.shape[2]
    shape = make_shape(B, Hq, Hkv, d, seq_len, stride)
    ws_bytes = lib().bsa_decode_workspace_size(ctypes.byref(shape), n_keep, block_size, n_splits)
    if ws_bytes == SIZE_MAX:
        raise ValueError("invalid decode arguments")
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check("sparse_decode_attn",
           lib().sparse_decode_attn_split(_ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), n_keep,
                                          ctypes.byref(shape), block_size, scale, _ptr(out),
                                          _ptr(lse), _ptr(workspace), workspace.numel(),
                                          n_splits, _stream(q.device)))
    return out, lse


def sparse_decode_partials(q, k, v, block_idx, seq_len, block_size=64, scale=0.0, n_splits=0,
                           workspace=None):
    """Step S4 alone: the split-K partial softmax states of sparse_decode_attn, written into
    `workspace` (uint8, allocated when None).  Returns the workspace."""
    import torch
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(block_idx, "block_idx", torch.int32, 3)
    B, Hq, d = q.shape
    Hkv, stride = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or block_idx.shape[:2] != (B, Hkv):
        raise ValueError("k, v and block_idx shapes disagree")
    n_keep = block_idx.shape[2]
    shape = make_shape(B, Hq, Hkv, d, seq_len, stride)
    ws_bytes = lib().bsa_decode_workspace_size(ctypes.byref(shape), n_keep, block_size, n_splits)
    if ws_bytes == SIZE_MAX:
        raise ValueError("invalid decode arguments")
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    _check("sparse_decode_partials",
           lib().sparse_decode_partials(_ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), n_keep,
                                        ctypes.byref(shape), block_size, scale, _ptr(workspace),
                                        workspace.numel(), n_splits, _stream(q.device)))
    return workspace


def sparse_decode_merge(workspace, batch, n_q_heads, n_kv_heads, head_dim, seq_len, n_keep,
                        block_size=64, n_splits=0, seq_stride=None, out=None, lse=None,
                        want_lse=True):
    """Step S5 alone: the exact merge of the partials sparse_decode_partials wrote with the
    same sizes.  Returns (out fp32 [B][Hq][d], lse fp32 [B][Hq] or None)."""
    import torch
    shape = make_shape(batch, n_q_heads, n_kv_heads, head_dim, seq_len,
                       seq_len if seq_stride is None else seq_stride)
    if out is None:
        out = torch.empty((batch, n_q_heads, head_dim), dtype=torch.float32,
                          device=workspace.device)
    if lse is None and want_lse:
        lse = torch.empty((batch, n_q_heads), dtype=torch.float32, device=workspace.device)
    _check("sparse_decode_merge",
           lib().sparse_decode_merge(ctypes.byref(shape), n_keep, block_size, n_splits,
                                     _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
                                     _stream(workspace.device)))
    return out, lse


def sparse_prefill_attn(q, k, v, k_cmp_sparse_f32, k_cmp_sparse_bf16, v_cmp_sparse_bf16,
                        k_cmp_dense_bf16, v_cmp_dense_bf16, prior_len, cfg=None, scale=0.0,
                        want_lse3=False, want_sel=False, out=None, workspace=None,
                        sink_logits=None):
    """Chunked prefill: q bf16 [B][C][Hq][d]; k, v bf16 [B][Hkv][stride][d] with the chunk's
    K/V at [prior_len, prior_len + C).  Returns (out fp32 [B][C][Hq][d], lse3, sel)."""
    import torch
    cfg = cfg or prefill_cfg()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    if cfg.indexer == INDEXER_F32:
        _need(k_cmp_sparse_f32, "k_cmp_sparse_f32", torch.float32, 4)
    for name, t in (("k_cmp_sparse_bf16", k_cmp_sparse_bf16),
                    ("v_cmp_sparse_bf16", v_cmp_sparse_bf16),
                    ("k_cmp_dense_bf16", k_cmp_dense_bf16), ("v_cmp_dense_bf16", v_cmp_dense_bf16)):
        _need(t, name, torch.bfloat16, 4)
    B, C, Hq, d = q.shape
    Hkv, stride = k.shape[1], k.shape[2]
    shape = make_shape(B, Hq, Hkv, d, prior_len, stride)
    E_s = num_blocks(prior_len, cfg.m_sparse)
    kk = min(cfg.top_k_sparse, E_s)
    n_tiles = -(-C // cfg.q_tile)
    ws_bytes = lib().bsa_prefill_workspace_size(ctypes.byref(shape), C, ctypes.byref(cfg))
    if ws_bytes == SIZE_MAX:
        raise ValueError("invalid prefill arguments")
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, C, Hq, d), dtype=torch.float32, device=q.device)
    lse3 = torch.empty((3, B, C, Hq), dtype=torch.float32, device=q.device) if want_lse3 else None
    sel = (torch.empty((B, n_tiles, Hkv, kk), dtype=torch.int32, device=q.device)
           if want_sel else None)
    _check("sparse_prefill_attn",
           lib().sparse_prefill_attn(_ptr(q), C, _ptr(k), _ptr(v), _ptr(k_cmp_sparse_f32),
                                     _ptr(k_cmp_sparse_bf16), _ptr(v_cmp_sparse_bf16),
                                     _ptr(k_cmp_dense_bf16), _ptr(v_cmp_dense_bf16),
                                     ctypes.byref(shape), ctypes.byref(cfg), scale,
                                     _ptr(_sink(sink_logits, Hq)), _ptr(out),
                                     _ptr(lse3), _ptr(sel), _ptr(workspace), workspace.numel(),
                                     _stream(q.device)))
    return out, lse3, sel


def _sink(t, Hq):
    """Per-head sink logits as a contiguous fp32 device tensor [Hq], or None."""
    import torch
    if t is None:
        return None
    _need(t, "sink_logits", torch.float32, 1)
    if t.shape[0] != Hq:
        raise ValueError(f"sink_logits must have {Hq} entries")
    return t


def _prefill_shape(q, k, prior_len, cfg):
    import torch
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    B, C, Hq, d = q.shape
    shape = make_shape(B, Hq, k.shape[1], d, prior_len, k.shape[2])
    n_tiles = -(-C // cfg.q_tile)
    kk = min(cfg.top_k_sparse, num_blocks(prior_len, cfg.m_sparse))
    return shape, n_tiles, kk


def select_prefill_entries(q, k, k_cmp_sparse_f32, k_cmp_sparse_bf16, prior_len, cfg=None,
                           sel=None, workspace=None):
    """The prefill's entry selection alone: sel int32 [B][n_tiles][Hkv][min(top_k, E_s)].
    k (bf16 [B][Hkv][stride][d]) only supplies the cache shape; of the two key streams only
    the one cfg.indexer names is read (the other may be None)."""
    import torch
    cfg = cfg or prefill_cfg()
    if cfg.indexer == INDEXER_F32:
        _need(k_cmp_sparse_f32, "k_cmp_sparse_f32", torch.float32, 4)
    else:
        _need(k_cmp_sparse_bf16, "k_cmp_sparse_bf16", torch.bfloat16, 4)
    shape, n_tiles, kk = _prefill_shape(q, k, prior_len, cfg)
    C = q.shape[1]
    ws_bytes = lib().bsa_prefill_workspace_size(ctypes.byref(shape), C, ctypes.byref(cfg))
    if ws_bytes == SIZE_MAX:
        raise ValueError("invalid prefill arguments")
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    if sel is None:
        sel = torch.empty((q.shape[0], n_tiles, k.shape[1], kk), dtype=torch.int32,
                          device=q.device)
    _check("select_prefill_entries",
           lib().select_prefill_entries(_ptr(q), C, _ptr(k_cmp_sparse_f32),
                                        _ptr(k_cmp_sparse_bf16), ctypes.byref(shape),
                                        ctypes.byref(cfg), _ptr(sel), _ptr(workspace),
                                        workspace.numel(), _stream(q.device)))
    return sel


def sparse_prefill_attn_selected(q, k, v, k_cmp_sparse_bf16, v_cmp_sparse_bf16, k_cmp_dense_bf16,
                                 v_cmp_dense_bf16, sel, prior_len, cfg=None, scale=0.0,
                                 want_lse3=False, out=None, sink_logits=None):
    """The prefill's three branches and their average over a given selection `sel`."""
    import torch
    cfg = cfg or prefill_cfg()
    _need(v, "v", torch.bfloat16, 4)
    for name, t in (("k_cmp_sparse_bf16", k_cmp_sparse_bf16),
                    ("v_cmp_sparse_bf16", v_cmp_sparse_bf16),
                    ("k_cmp_dense_bf16", k_cmp_dense_bf16), ("v_cmp_dense_bf16", v_cmp_dense_bf16)):
        _need(t, name, torch.bfloat16, 4)
    _need(sel, "sel", torch.int32, 4)
    shape, n_tiles, kk = _prefill_shape(q, k, prior_len, cfg)
    B, C, Hq, d = q.shape
    if tuple(sel.shape) != (B, n_tiles, k.shape[1], kk):
        raise ValueError(f"sel must be [{B}, {n_tiles}, {k.shape[1]}, {kk}]")
    if out is None:
        out = torch.empty((B, C, Hq, d), dtype=torch.float32, device=q.device)
    lse3 = torch.empty((3, B, C, Hq), dtype=torch.float32, device=q.device) if want_lse3 else None
    _check("sparse_prefill_attn_selected",
           lib().sparse_prefill_attn_selected(_ptr(q), C, _ptr(k), _ptr(v),
                                              _ptr(k_cmp_sparse_bf16), _ptr(v_cmp_sparse_bf16),
                                              _ptr(k_cmp_dense_bf16), _ptr(v_cmp_dense_bf16),
                                              _ptr(sel), ctypes.byref(shape), ctypes.byref(cfg),
                                              scale, _ptr(_sink(sink_logits, Hq)), _ptr(out),
                                              _ptr(lse3), _stream(q.device)))
    return out, lse3


def quantize_kv_fp8(x, seq_len, block_size=64, summary_stride=0, out=None, scales=None):
    """x bf16 [B][H][stride][d] -> (E4M3 codes uint8 [B][H][stride][d], fp32 scales [B][H][S]),
    S = summary_stride or ceil(seq_len / block_size); one scale per block."""
    import torch
    _need(x, "x", torch.bfloat16, 4)
    B, H, stride, d = x.shape
    S = summary_stride or num_blocks(seq_len, block_size)
    if out is None:
        out = torch.zeros((B, H, stride, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, S), dtype=torch.float32, device=x.device)
    shape = make_shape(B, H, H, d, seq_len, stride, summary_stride)
    _check("quantize_kv_fp8", lib().quantize_kv_fp8(_ptr(x), ctypes.byref(shape), block_size,
                                                    _ptr(out), _ptr(scales), _stream(x.device)))
    return out, scales


def sparse_decode_attn_fp8(q, k8, v8, k_scales, v_scales, block_idx, seq_len, block_size=64,
                           scale=0.0, out=None, lse=None, workspace=None, want_lse=True):
    """sparse_decode_attn over an E4M3 cache from quantize_kv_fp8 (k8, v8 uint8
    [B][Hkv][stride][d], scales fp32 [B][Hkv][S])."""
    import torch
    _need(q, "q", torch.bfloat16, 3)
    for name, t in (("k8", k8), ("v8", v8)):
        _need(t, name, torch.uint8, 4)
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        _need(t, name, torch.float32, 3)
    _need(block_idx, "block_idx", torch.int32, 3)
    B, Hq, d = q.shape
    Hkv, stride = k8.shape[1], k8.shape[2]
    if tuple(v8.shape) != tuple(k8.shape) or tuple(v_scales.shape) != tuple(k_scales.shape):
        raise ValueError("k/v shapes disagree")
    n_keep = block_idx.shape[2]
    shape = make_shape(B, Hq, Hkv, d, seq_len, stride, k_scales.shape[2])
    ws_bytes = lib().bsa_decode_workspace_size(ctypes.byref(shape), n_keep, block_size, 0)
    if ws_bytes == SIZE_MAX:
        raise ValueError("invalid decode arguments")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    _check("sparse_decode_attn_fp8",
           lib().sparse_decode_attn_fp8(_ptr(q), _ptr(k8), _ptr(v8), _ptr(k_scales),
                                        _ptr(v_scales), _ptr(block_idx), n_keep,
                                        ctypes.byref(shape), block_size, scale, _ptr(out),
                                        _ptr(lse), _ptr(workspace), workspace.numel(),
                                        _stream(q.device)))
    return out, lse


def decode_step(q, k, v, summaries, seq_len, block_size=64, n_sink=1, n_local=2, top_k=-1,
                keep_ratio=0.0, scale=0.0, **adaptive):
    """select_blocks then sparse_decode_attn (the per-token hot path); `adaptive` takes the
    select_blocks keywords adaptive, keep_ratio_max and anchor_margin."""
    idx, _ = select_blocks(q, summaries, seq_len, block_size, n_sink, n_local, top_k, keep_ratio,
                           **adaptive)
    out, lse = sparse_decode_attn(q, k, v, idx, seq_len, block_size, scale)
    return out, lse, idx


def decode_loop_step(q, k_new, v_new, k_cache, v_cache, summaries, seq_len, block_size=64,
                     n_sink=1, n_local=2, top_k=-1, keep_ratio=0.0, scale=0.0, block_idx=None,
                     out=None, lse=None, workspace=None):
    """One generated token: append its K/V at seq_len, refresh the summary of the block it
    lands in (or opens), then select and attend over seq_len + n tokens in one
    sparse_decode_step call.  summaries fp32 or bf16 [B][Hkv][S][d] with
    S >= ceil(capacity / block_size).  Returns (out, lse, idx)."""
    n = k_new.shape[2]
    append_kv(k_new, v_new, k_cache, v_cache, seq_len, block_size, summaries)
    return sparse_decode_step(q, k_cache, v_cache, summaries, seq_len + n, block_size, n_sink,
                              n_local, top_k, keep_ratio, scale, block_idx=block_idx, out=out,
                              lse=lse, workspace=workspace)


def build_compressed_streams(k, v, prior_len, cfg=None, want_f32=None):
    """The prefill's pooled streams over the prior tokens: bf16 keys and values at m_sparse
    (plus the fp32 keys when want_f32, by default when cfg.indexer is INDEXER_F32; else None),
    bf16 keys and values at m_dense (all via build_block_summaries)."""
    cfg = cfg or prefill_cfg()
    if want_f32 is None:
        want_f32 = cfg.indexer == INDEXER_F32
    k4f, k4b = build_block_summaries(k, prior_len, cfg.m_sparse, want_f32=want_f32,
                                     want_bf16=True)
    _, v4b = build_block_summaries(v, prior_len, cfg.m_sparse, want_f32=False, want_bf16=True)
    _, k128b = build_block_summaries(k, prior_len, cfg.m_dense, want_f32=False, want_bf16=True)
    _, v128b = build_block_summaries(v, prior_len, cfg.m_dense, want_f32=False, want_bf16=True)
    return k4f, k4b, v4b, k128b, v128b


def prefill_step(q, k, v, prior_len, cfg=None, scale=0.0, want_lse3=False, want_sel=False,
                 streams=None, sink_logits=None):
    """Chunked prefill: pooled streams (unless given), then sparse_prefill_attn."""
    cfg = cfg or prefill_cfg()
    if streams is None:
        streams = build_compressed_streams(k, v, prior_len, cfg)
    return sparse_prefill_attn(q, k, v, *streams, prior_len, cfg=cfg, scale=scale,
                               want_lse3=want_lse3, want_sel=want_sel, sink_logits=sink_logits)
