"""The causal (and sliding-window) tile skip of the T=8192 prefill, pinned by
the matrix-core instruction counter.

A wave of the 8-wave prefill owns 32 query rows and visits a 128-key tile
only when some row of its block sees some key of the tile (the block-skip
rule of the Ch. 11 "Attention" page, section 11.8.3, with exact bounds); each
visited tile costs 64 MFMAs (32 for the scores, 32 for P.V).  The count of
visited (wave, tile) pairs has a closed form, checked here against a brute
force over the mask definition, and the MFMA count it implies must equal
SQ_INSTS_MFMA of the committed rocprofv3 counter runs, exactly: a kernel that
visited extra tiles would show up here, not only as lost speed."""
import json

import numpy as np
import pytest

import bench

ROWS, BN, MFMA_PER_TILE = 32, 128, 64


def closed_form_tiles(T, window=0):
    """Visited (wave, tile) pairs of one head: a wave's rows r0..r0+31 see
    keys max(0, r - W + 1)..r, so it visits tiles floor(first / BN) ..
    ceil(last_end / BN) - 1."""
    total = 0
    for r0 in range(0, T, ROWS):
        last = min(T, r0 + ROWS)           # one past the block's last visible key
        first = max(0, r0 - window + 1) if window else 0
        total += -(-last // BN) - first // BN
    return total


def brute_force_tiles(T, window=0):
    """The same count from the mask definition itself: tile t is visited by
    the block iff some (row, key) pair in it is visible."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    vis = j <= i
    if window:
        vis &= j > i - window
    n = 0
    for r0 in range(0, T, ROWS):
        blk = vis[r0:r0 + ROWS]
        for t in range(-(-T // BN)):
            n += bool(blk[:, t * BN:(t + 1) * BN].any())
    return n


@pytest.mark.parametrize("T,window", [(256, 0), (1000, 0), (1024, 100), (2048, 700), (1536, 1)])
def test_closed_form_matches_the_mask(T, window):
    assert closed_form_tiles(T, window) == brute_force_tiles(T, window)


def test_causal_count_is_the_known_total():
    # 8192 rows: 8320 visited (wave, tile) pairs per head, 32 heads
    assert closed_form_tiles(8192) == 8320
    assert 32 * 8320 * MFMA_PER_TILE == 17_039_360


@pytest.mark.parametrize("name,window", [("prefill_bf16_T8192_D128_gqa", 0),
                                         ("window_prefill_bf16_T8192_W4096_D128_gqa", 4096)])
def test_mfma_counter_equals_closed_form(name, window):
    rec = json.loads((bench.PROFILES / f"{name}_counters.json").read_text())
    _, files = bench.KERNELS[name]
    csrc = bench.ROOT / "transformer_scaled_dot_flash_amd" / "csrc"
    assert rec["source_sha256"] == bench.source_digest([csrc / f for f in files]), "re-take the counters"
    want = 32 * closed_form_tiles(8192, window) * MFMA_PER_TILE
    assert rec["counters_per_dispatch"]["SQ_INSTS_MFMA"] == want
