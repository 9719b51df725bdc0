"""The C ABI library loads, exports every entry point of include/bsa.h, and its
host-side logic (counts, workspace sizes, argument checks) behaves.  No GPU:
every call here returns before any launch."""
import ctypes
import os
import re

import pytest

import long_context_block_summary_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsa.LIB_PATH):
        pytest.fail("libbsa.so is not built")
    return bsa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    for must in ("build_block_summaries", "select_blocks", "sparse_decode_attn",
                 "sparse_prefill_attn"):
        assert must in names
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_counts(L):
    assert bsa.num_blocks(1_000_000, 4) == 250_000
    assert bsa.num_blocks(1_000_000, 128) == 7813
    assert bsa.num_blocks(-1, 4) == -1 and bsa.num_blocks(5, 0) == -1
    for nb, r, k in [(512, 0.15, 74), (2048, 0.10, 202), (16384, 0.10, 1635)]:
        assert bsa.num_kept(nb, bsa.select_cfg(keep_ratio=r)) == k + 3
        assert bsa.num_kept(nb, bsa.select_cfg(top_k=k)) == k + 3
    assert bsa.num_kept(3, bsa.select_cfg(top_k=5)) == 3
    assert bsa.num_kept(16, bsa.select_cfg(top_k=100)) == 16
    assert bsa.num_kept(16, bsa.select_cfg(n_sink=-1)) == -1


def test_workspace_sizes(L):
    sh = bsa.make_shape(4, 64, 8, 128, 131072, 131072)
    cfg = bsa.select_cfg(top_k=202)
    assert L.bsa_select_workspace_size(ctypes.byref(sh), ctypes.byref(cfg)) == 4 * 8 * 2048 * 4
    ws1 = L.bsa_decode_workspace_size(ctypes.byref(sh), 205, 64, 1)
    assert ws1 == 32 * 1 * 8 * 130 * 4   # (o, m, l) split partials
    assert L.bsa_decode_workspace_size(ctypes.byref(sh), 205, 64, 0) >= ws1
    bad = bsa.make_shape(4, 63, 8, 128, 10, 10)
    assert L.bsa_decode_workspace_size(ctypes.byref(bad), 5, 64, 0) == bsa.SIZE_MAX


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(L.bsa_status_string(s), bytes)


def test_argument_checks_launch_nothing(L):
    sh = bsa.make_shape(1, 4, 4, 128, 1024, 1024)
    cfg = bsa.select_cfg(top_k=4)
    fake = ctypes.c_void_p(0x1000)
    # NULL input / outputs
    assert L.build_block_summaries(None, ctypes.byref(sh), 64, fake, None, None) == -1
    assert L.build_block_summaries(fake, ctypes.byref(sh), 64, None, None, None) == -1
    # misaligned pointer
    assert L.build_block_summaries(ctypes.c_void_p(0x1002), ctypes.byref(sh), 64, fake, None,
                                   None) == -1
    # unsupported head_dim
    sh96 = bsa.make_shape(1, 4, 4, 96, 1024, 1024)
    assert L.build_block_summaries(fake, ctypes.byref(sh96), 64, fake, None, None) == -2
    # Hq % Hkv != 0
    bad = bsa.make_shape(1, 6, 4, 128, 1024, 1024)
    assert L.select_blocks(fake, fake, ctypes.byref(bad), ctypes.byref(cfg), fake, None, fake,
                           1 << 20, None) == -1
    # workspace too small
    assert L.select_blocks(fake, fake, ctypes.byref(sh), ctypes.byref(cfg), fake, None, fake, 8,
                           None) == -3
    # decode: block size other than 64 is unsupported, n_keep beyond nb is invalid
    assert L.sparse_decode_attn(fake, fake, fake, fake, 4, ctypes.byref(sh), 32, 0.0, fake, None,
                                fake, 1 << 20, None) == -2
    assert L.sparse_decode_attn(fake, fake, fake, fake, 17, ctypes.byref(sh), 64, 0.0, fake,
                                None, fake, 1 << 20, None) == -1
    assert L.sparse_decode_attn(fake, fake, fake, fake, 0, ctypes.byref(sh), 64, 0.0, fake, None,
                                fake, 1 << 20, None) == -1
    g32 = bsa.make_shape(1, 32, 1, 128, 1024, 1024)
    assert L.sparse_decode_attn(fake, fake, fake, fake, 4, ctypes.byref(g32), 64, 0.0, fake,
                                None, fake, 1 << 20, None) == -2
    assert L.sparse_decode_attn(fake, fake, fake, fake, 4, ctypes.byref(sh), 64, 0.0, fake, None,
                                fake, 16, None) == -3
    # stride below seq_len
    short = bsa.make_shape(1, 4, 4, 128, 1024, 1000)
    assert L.sparse_decode_attn(fake, fake, fake, fake, 4, ctypes.byref(short), 64, 0.0, fake,
                                None, fake, 1 << 20, None) == -1


def test_decode_step_calls_check_arguments(L):
    """S4 (sparse_decode_partials) and S5 (sparse_decode_merge) alone: the checks of
    sparse_decode_attn_split, and their own NULL / alignment checks."""
    sh = bsa.make_shape(1, 4, 4, 128, 1024, 1024)
    fake = ctypes.c_void_p(0x1000)
    ws = 1 << 20
    P, M = L.sparse_decode_partials, L.sparse_decode_merge
    assert P(None, fake, fake, fake, 4, ctypes.byref(sh), 64, 0.0, fake, ws, 0, None) == -1
    assert P(fake, fake, fake, None, 4, ctypes.byref(sh), 64, 0.0, fake, ws, 0, None) == -1
    assert P(ctypes.c_void_p(0x1004), fake, fake, fake, 4, ctypes.byref(sh), 64, 0.0, fake, ws, 0,
             None) == -1
    assert P(fake, fake, fake, fake, 4, ctypes.byref(sh), 32, 0.0, fake, ws, 0, None) == -2
    assert P(fake, fake, fake, fake, 17, ctypes.byref(sh), 64, 0.0, fake, ws, 0, None) == -1
    assert P(fake, fake, fake, fake, 4, ctypes.byref(sh), 64, 0.0, fake, 16, 0, None) == -3
    assert P(fake, fake, fake, fake, 4, ctypes.byref(sh), 64, 0.0, None, ws, 0, None) == -1
    assert P(fake, fake, fake, fake, 4, ctypes.byref(sh), 64, 0.0, fake, ws, -1, None) == -1
    assert M(ctypes.byref(sh), 4, 64, 0, fake, ws, None, None, None) == -1
    assert M(ctypes.byref(sh), 4, 64, 0, fake, ws, ctypes.c_void_p(0x1008), None, None) == -1
    assert M(ctypes.byref(sh), 4, 64, 0, fake, 16, fake, None, None) == -3
    assert M(ctypes.byref(sh), 4, 64, 0, None, ws, fake, None, None) == -1
    assert M(ctypes.byref(sh), 0, 64, 0, fake, ws, fake, None, None) == -1
    g32 = bsa.make_shape(1, 32, 1, 128, 1024, 1024)
    assert M(ctypes.byref(g32), 4, 64, 0, fake, ws, fake, None, None) == -2
    assert M(None, 4, 64, 0, fake, ws, fake, None, None) == -1
    # a kv head's rows beyond 32-bit byte offsets: bf16 from 2^24 + 1 tokens at d = 128,
    # FP8 from 2^25 + 1
    for n, code in ((1 << 24, -3), ((1 << 24) + 64, -2)):
        big = bsa.make_shape(1, 4, 4, 128, n, n)
        assert P(fake, fake, fake, fake, 4, ctypes.byref(big), 64, 0.0, fake, 16, 0, None) == code
    for n, code in ((1 << 25, -3), ((1 << 25) + 64, -2)):
        big = bsa.make_shape(1, 4, 4, 128, n, n)
        assert L.sparse_decode_attn_fp8(fake, fake, fake, fake, fake, fake, 4, ctypes.byref(big),
                                        64, 0.0, fake, None, fake, 16, None) == code


def test_decode_step_checks_arguments(L):
    """sparse_decode_step: NULL / alignment, adaptive selection refused, workspace size."""
    sh = bsa.make_shape(1, 4, 4, 128, 1024, 1024)
    cfg = bsa.select_cfg(64, 1, 2, 4)
    fake = ctypes.c_void_p(0x1000)
    ws = L.bsa_decode_step_workspace_size(ctypes.byref(sh), ctypes.byref(cfg))
    assert 0 < ws < 1 << 30
    S = L.sparse_decode_step
    args = lambda **kw: [kw.get("q", fake), fake, fake, fake, ctypes.byref(sh),
                         ctypes.byref(kw.get("cfg", cfg)), kw.get("idx", fake), 0.0,
                         kw.get("out", fake), None, kw.get("ws", fake), kw.get("ws_bytes", ws),
                         None]
    assert S(*args(q=None)) == -1
    assert S(*args(idx=None)) == -1
    assert S(*args(out=ctypes.c_void_p(0x1004))) == -1
    assert S(*args(ws=None)) == -1
    assert S(*args(ws_bytes=ws - 1)) == -3
    adaptive = bsa.select_cfg(64, 1, 2, -1, 0.1, True, 0.2, 0.0)
    assert S(*args(cfg=adaptive)) == -2


def test_select_cfg_summary_type_checked(L):
    """bsa_select_cfg.summaries_bf16 takes 0 (fp32 summaries) or 1 (bf16); anything else is
    an invalid config, refused before any launch."""
    fake = ctypes.c_void_p(0x1000)
    sh = bsa.make_shape(1, 8, 2, 128, 4096, 4096)
    for flag, want in ((0, 67), (1, 67), (2, -1), (-1, -1)):
        cfg = bsa.select_cfg(top_k=64)
        cfg.summaries_bf16 = flag
        assert L.bsa_num_kept(200, ctypes.byref(cfg)) == want
        if want < 0:
            assert L.select_blocks(fake, fake, ctypes.byref(sh), ctypes.byref(cfg), fake, None,
                                   fake, 1 << 20, None) == -1


def test_prefill_argument_checks_launch_nothing(L):
    fake = ctypes.c_void_p(0x1000)
    pc = bsa.prefill_cfg()
    sh = bsa.make_shape(1, 32, 8, 128, 4096, 4096 + 128)
    # NULL q; chunk overruns the cache capacity; bad tile shape; workspace too small
    assert L.select_prefill_entries(None, 128, fake, fake, ctypes.byref(sh), ctypes.byref(pc), fake,
                                    fake, 1 << 30, None) == -1
    assert L.select_prefill_entries(fake, 256, fake, fake, ctypes.byref(sh), ctypes.byref(pc), fake,
                                    fake, 1 << 30, None) == -1
    odd = bsa.prefill_cfg(q_tile=48)
    assert L.select_prefill_entries(fake, 128, fake, fake, ctypes.byref(sh), ctypes.byref(odd), fake,
                                    fake, 1 << 30, None) == -2
    assert L.select_prefill_entries(fake, 128, fake, fake, ctypes.byref(sh), ctypes.byref(pc),
                                    fake, fake, 64, None) == -3
    # the indexer's keys: the stream cfg.indexer names must be given, the other may be NULL;
    # an unknown indexer is invalid
    f32 = bsa.prefill_cfg(indexer=bsa.INDEXER_F32)
    # (sparse_prefill_attn always reads the bf16 keys: branch A attends them)
    for cfg, f, b, w_sel, w_all in ((pc, None, fake, -3, -3), (pc, fake, None, -1, -1),
                                    (f32, fake, None, -3, -1), (f32, None, fake, -1, -1),
                                    (bsa.prefill_cfg(indexer=2), fake, fake, -1, -1)):
        assert L.select_prefill_entries(fake, 128, f, b, ctypes.byref(sh), ctypes.byref(cfg),
                                        fake, fake, 64, None) == w_sel
        assert L.sparse_prefill_attn(fake, 128, fake, fake, f, b, fake, fake, fake,
                                     ctypes.byref(sh), ctypes.byref(cfg), 0.0, None, fake, None,
                                     None, fake, 64, None) == w_all
    # attention over a given selection: NULL selection, misaligned stream
    args = [fake, 128, fake, fake, fake, fake, fake, fake]
    assert L.sparse_prefill_attn_selected(*args, None, ctypes.byref(sh), ctypes.byref(pc), 0.0,
                                          None, fake, None, None) == -1
    args[4] = ctypes.c_void_p(0x1004)
    assert L.sparse_prefill_attn_selected(*args, fake, ctypes.byref(sh), ctypes.byref(pc), 0.0,
                                          None, fake, None, None) == -1
    # unknown combination mode
    args[4] = fake
    bad_mode = bsa.prefill_cfg(combine=2)
    assert L.sparse_prefill_attn_selected(*args, fake, ctypes.byref(sh), ctypes.byref(bad_mode),
                                          0.0, None, fake, None, None) == -1
    # more selected entries than the kernel keeps in LDS; compressed stream too long
    big_k = bsa.prefill_cfg(top_k_sparse=8192)
    sh_long = bsa.make_shape(1, 32, 8, 128, 1 << 16, (1 << 16) + 128)
    assert L.sparse_prefill_attn(fake, 128, fake, fake, fake, fake, fake, fake, fake,
                                 ctypes.byref(sh_long), ctypes.byref(big_k), 0.0, None, fake,
                                 None, None, fake, 1 << 40, None) == -2
    sh_huge = bsa.make_shape(1, 32, 8, 128, 1 << 20, (1 << 20) + 128)
    assert L.sparse_prefill_attn(fake, 128, fake, fake, fake, fake, fake, fake, fake,
                                 ctypes.byref(sh_huge), ctypes.byref(pc), 0.0, None, fake,
                                 None, None, fake, 1 << 40, None) == -2


def test_product_path_has_no_oracle_import():
    pkg = os.path.join(ROOT, "long_context_block_summary_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "oracle.h" not in text, f


def test_loop_argument_checks_launch_nothing(L):
    fake = ctypes.c_void_p(0x1000)
    sh = bsa.make_shape(1, 4, 4, 128, 100, 128)
    # append past the capacity; negative count; misaligned cache
    assert L.append_kv(fake, fake, fake, fake, ctypes.byref(sh), 29, 64, None, None, None) == -1
    assert L.append_kv(fake, fake, fake, fake, ctypes.byref(sh), -1, 64, None, None, None) == -1
    assert L.append_kv(fake, fake, ctypes.c_void_p(0x1008), fake, ctypes.byref(sh), 1, 64, None,
                       None, None) == -1
    # refresh with a summary stride below the blocks after the append (100 + 29 -> 3 blocks)
    two = bsa.make_shape(1, 4, 4, 128, 100, 256, 2)
    assert L.append_kv(fake, fake, fake, fake, ctypes.byref(two), 29, 64, fake, None, None) == -1
    assert L.append_kv(fake, fake, fake, fake, ctypes.byref(two), 28, 0, fake, None, None) == -1
    # first token beyond seq_len; summary stride below the blocks in use
    assert L.update_block_summaries(fake, ctypes.byref(sh), 64, 101, fake, None, None) == -1
    narrow = bsa.make_shape(1, 4, 4, 128, 100, 128, 1)
    assert L.update_block_summaries(fake, ctypes.byref(narrow), 64, 0, fake, None, None) == -1
    cfg = bsa.select_cfg(top_k=1)
    assert L.select_blocks(fake, fake, ctypes.byref(narrow), ctypes.byref(cfg), fake, None, fake,
                           1 << 20, None) == -1
    # nothing to update is a no-op
    assert L.update_block_summaries(fake, ctypes.byref(sh), 64, 100, fake, None, None) == 0


def test_keep_ratio_counts_equal_the_oracle(L, orc):
    """The kept count and the adaptive bounds follow the oracle's rounding of the ratio as
    given (floor(r * nb + 0.5) in double), including ratios whose float value would round
    the other way: (5, 0.7), (10, 0.35), (10, 0.45), (5, 0.9)."""
    import numpy as np
    for nb, r, kept in ((5, 0.7, 4), (10, 0.35, 4), (10, 0.45, 5), (5, 0.9, 5)):
        assert orc.num_kept(nb, 1, 2, -1, r) == kept
        assert bsa.num_kept(nb, bsa.select_cfg(keep_ratio=r)) == kept
        w, _, _ = orc.adaptive_bounds(nb, 1, 2, r, r)
        assert bsa.num_kept(nb, bsa.select_cfg(keep_ratio=r, adaptive=True,
                                               keep_ratio_max=r)) == w == kept
    ratios = [round(0.05 * i, 2) for i in range(1, 20)]
    for sink, local in ((1, 2), (0, 1), (2, 0)):
        for r in ratios:
            want = np.array([orc.num_kept(nb, sink, local, -1, r) for nb in range(1, 5001)])
            cfg = bsa.select_cfg(n_sink=sink, n_local=local, keep_ratio=r)
            got = np.array([L.bsa_num_kept(nb, ctypes.byref(cfg)) for nb in range(1, 5001)])
            assert np.array_equal(got, want), (sink, local, r)
        for lo, hi in zip(ratios[:-3], ratios[3:]):
            cfg = bsa.select_cfg(n_sink=sink, n_local=local, keep_ratio=lo, adaptive=True,
                                 keep_ratio_max=hi)
            lo_cfg = bsa.select_cfg(n_sink=sink, n_local=local, keep_ratio=lo, adaptive=True,
                                    keep_ratio_max=lo)
            for nb in range(1, 5001, 7):
                w, k_lo, k_hi = orc.adaptive_bounds(nb, sink, local, lo, hi)
                assert L.bsa_num_kept(nb, ctypes.byref(cfg)) == w, (nb, lo, hi)
                assert L.bsa_num_kept(nb, ctypes.byref(lo_cfg)) == w - k_hi + k_lo, (nb, lo)


def test_prefill_rejects_rows_beyond_32bit_offsets(L):
    """The attention addresses the dense stream's rows and a tile's window rows by 32-bit
    byte offsets (256-byte rows): E_d and min(window + q_tile, P + C) are bounded by 2^24."""
    fake = ctypes.c_void_p(0x1000)
    S = L.select_prefill_entries

    def call(P, C, **kw):
        sh = bsa.make_shape(1, 32, 8, 128, P, P + C)
        pc = bsa.prefill_cfg(**kw)
        return S(fake, C, fake, fake, ctypes.byref(sh), ctypes.byref(pc), fake, fake, 64, None)

    # dense stream: 2^24 entries pass the checks (then the workspace is too small), one more
    # is unsupported
    assert call(1 << 24, 128, m_sparse=256, m_dense=1) == -3
    assert call((1 << 24) + 1, 128, m_sparse=256, m_dense=1) == -2
    # window rows: min(window + q_tile, P + C)
    assert call(1 << 24, 128, m_sparse=256, window=(1 << 24) - 64) == -3
    assert call(1 << 24, 128, m_sparse=256, window=(1 << 24) - 63) == -2
    assert call(1 << 20, 128, m_sparse=256, window=1 << 30) == -3  # capped by P + C


def test_noalloc_step_checks_before_any_device_call(L):
    """sparse_decode_step_noalloc checks its arguments (and the scratch limit) before it
    touches the device: an invalid shape or config is BSA_INVALID_ARG, a step whose
    workspace exceeds the static scratch BSA_UNSUPPORTED."""
    fake = ctypes.c_void_p(0x1000)
    F = L.sparse_decode_step_noalloc
    F.argtypes = [ctypes.c_void_p] * 4 + [ctypes.POINTER(bsa.bsa_shape),
                                          ctypes.POINTER(bsa.bsa_select_cfg), ctypes.c_void_p,
                                          ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]
    F.restype = ctypes.c_int
    cfg = bsa.select_cfg(top_k=304)
    bad = bsa.make_shape(1, 6, 4, 128, 1024, 1024)        # Hq % Hkv != 0
    assert F(fake, fake, fake, fake, ctypes.byref(bad), ctypes.byref(cfg), fake, 0.0, fake, None,
             None) == -1
    assert F(fake, fake, fake, fake, None, ctypes.byref(cfg), fake, 0.0, fake, None, None) == -1
    neg = bsa.select_cfg(n_sink=-1)
    ok = bsa.make_shape(1, 4, 4, 128, 1024, 1024)
    assert F(fake, fake, fake, fake, ctypes.byref(ok), ctypes.byref(neg), fake, 0.0, fake, None,
             None) == -1
    big = bsa.make_shape(256, 64, 8, 128, 131072, 131072)
    assert L.bsa_decode_step_workspace_size(ctypes.byref(big), ctypes.byref(cfg)) > 16 << 20
    assert F(fake, fake, fake, fake, ctypes.byref(big), ctypes.byref(cfg), fake, 0.0, fake, None,
             None) == -2
