"""Work and byte accounting of the workloads, pinned to the pages' arithmetic."""
import math
from pathlib import Path

import pytest

from transformer_scaled_dot_flash_amd.workloads import BY_ORDINAL, WORKLOADS, Workload

GOLDEN = Path(__file__).resolve().parent / "golden" / "memory_arithmetic.txt"


def _golden():
    out = {}
    for ln in GOLDEN.read_text().splitlines():
        if ln.strip() and not ln.startswith("#"):
            name, val, _src = ln.split()
            out[name] = int(val)
    return out


def test_kv_cache_bytes_match_the_pages():
    g = _golden()
    # K and V, fp16, per token per layer: 2 * n_kv * head_dim * 2 bytes
    for name, n_kv in [("mha_g32", 32), ("gqa_g8", 8), ("mqa_g1", 1)]:
        w = Workload("t", 9, "decode", 1, 32, n_kv, 1, 1, 128, False, "bf16", 0.1)
        per_token = w.bytes() - 2 * 2 * 32 * 128  # drop Q and O
        assert per_token == g[f"kv_per_token_{name}"]
        w4k = Workload("t", 9, "decode", 1, 32, n_kv, 1, 4096, 128, False, "bf16", 0.1)
        assert w4k.bytes() - 2 * 2 * 32 * 128 == g[f"kv_4096_tokens_{name}"]
    assert g["kv_per_token_llama3_8b"] == g["kv_per_token_gqa_g8"]
    assert 16 * g["kv_per_token_llama3_8b"] == g["kv_block_16_tokens"]
    assert 32 * g["kv_block_16_tokens"] == g["kv_32_blocks"]


def test_score_matrix_sizes_match_the_pages():
    g = _golden()
    assert 4 * 2048 * 2048 == g["score_matrix_f32_T2048"]
    assert 4 * 8192 * 8192 == g["score_matrix_f32_T8192"]
    assert 32 * 8192 * 8192 * 2 == g["scores_fp16_32heads_8k"]


def test_flop_count_matches_the_table():
    """AIInfraGuide section 11.1: QK^T and PV cost 2 N^2 d each, so the full
    (non-causal) attention core is 4 N^2 d per head."""
    N, d = 512, 64
    w = Workload("t", 9, "prefill", 1, 1, 1, N, N, d, False, "bf16", 0.125)
    assert w.flops() == 4 * N * N * d
    wc = Workload("t", 9, "prefill", 1, 1, 1, N, N, d, True, "bf16", 0.125)
    assert wc.flops() == 4 * d * N * (N + 1) // 2


def test_headline_workloads():
    c4 = BY_ORDINAL[4]
    assert c4.flops() == 549_822_922_752
    assert c4.bytes() == 167_772_160
    c5 = BY_ORDINAL[5]
    assert c5.bytes() == 1_074_790_400
    assert c5.bytes() - 2 * 2 * 64 * 32 * 128 == 64 * 4096 * 4096  # 64 seqs x 4096 tokens x 4 KiB
    assert c5.flops() == 4_294_967_296
    assert BY_ORDINAL[1].scale == 0.125
    assert BY_ORDINAL[4].scale == float.fromhex("0x1.6a09e60000000p-4")  # float32(1/sqrt(128))


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_scale_is_float32(name):
    w = WORKLOADS[name]
    import numpy as np
    assert float(np.float32(w.scale)) == w.scale
    assert abs(w.scale - 1.0 / math.sqrt(w.D)) < 1e-7
