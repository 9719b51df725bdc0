"""The benchmark's work accounting, which every roofline fraction rests on, checked against
figures written out term by term and against the sizes the pages print.  CPU only."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_block_summary_amd import synth  # noqa: E402
from test_oracle_pins import golden  # noqa: E402


def test_kv_bytes_per_token_match_the_pages():
    g = golden()
    per_tok = bench.kv_bytes_per_token(32, 128, 2)          # 32 layers x 2 x 128 dims x 2 bytes
    assert per_tok == 16384
    for key, n_tok in (("kv_bytes_per_token_fp16", 1), ("kv_bytes_200k_fp16", 200_000),
                       ("kv_bytes_1m_fp16", 1_000_000)):
        val, kind = g[key]
        assert kind == "approx" and abs(per_tok * n_tok - val) <= 0.05 * val, key
    one_layer = 1_000_000 * bench.kv_bytes_per_token(1, 128, 2)
    assert abs(one_layer - g["kv_bytes_one_layer_1m"][0]) <= 0.01 * g["kv_bytes_one_layer_1m"][0]
    assert abs(61 * one_layer - g["kv_bytes_61_layers_1m"][0]) <= 0.02 * g["kv_bytes_61_layers_1m"][0]


# per decode workload: kept K and V (kept blocks x 64 tokens x d x 2 bytes x 2) + fp32
# summaries of every block + q (bf16) + out (fp32) + lse (fp32) + the int32 kept lists
STEP_BYTES = {
    # 8 x 8 x (77 x 32768 + 512 x 512) + 8 x 32 x (256 + 512 + 4) + 8 x 8 x 77 x 4
    "gqa32k": 178_475_264,
    # 4 x 8 x (205 x 32768 + 2048 x 512) + 4 x 64 x 772 + 4 x 8 x 205 x 4
    "long128k": 248_736_384,
    # 4 x 8 x (307 x 32768 + 2048 x 512) + 4 x 64 x 772 + 4 x 8 x 307 x 4
    "long128k_15": 355_704_192,
    # 1 x 8 x (1638 x 32768 + 16384 x 512) + 1 x 128 x 772 + 1 x 8 x 1638 x 4
    "ctx1m": 496_651_968,
}


@pytest.mark.parametrize("name", sorted(STEP_BYTES))
def test_decode_step_bytes(name):
    cfg = synth.CONFIGS[name]
    n_keep = cfg.top_k + cfg.n_sink + cfg.n_local
    assert bench.step_bytes(cfg, n_keep) == STEP_BYTES[name]
    sel, att = bench.decode_bytes(cfg, n_keep)
    q = cfg.batch * cfg.n_q_heads * cfg.head_dim * 2
    nb = cfg.seq_len // 64
    assert sel == cfg.batch * cfg.n_kv_heads * nb * cfg.head_dim * 4 + q
    assert sel + att - q == STEP_BYTES[name]


def test_partials_bytes():
    # the split-K kernel alone: kept K and V + q + the kept lists (its partials are scratch)
    cfg = synth.CONFIGS["long128k_15"]
    assert bench.partials_bytes(cfg, 307) == 4 * 8 * 307 * 32768 + 4 * 64 * 128 * 2 + 4 * 8 * 307 * 4
    assert bench.partials_bytes(cfg, 307) == 322_017_664


def test_prefill_flops():
    # 2 flops per multiply-add, QK^T and PV, over 2048 selected + 2048 dense + 128 window
    # entries for 2048 queries x 32 heads at d = 128
    cfg = synth.CONFIGS["prefill256k"]
    assert bench.prefill_flops(cfg, 2048, 2048) == 2 * 2 * 128 * 2048 * 32 * (2048 + 2048 + 128)
    assert bench.prefill_flops(cfg, 2048, 2048) == 141_733_920_768
