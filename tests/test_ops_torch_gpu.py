"""The torch front end (ops_torch) allocates outputs and calls the C ABI:
each function must give bit for bit what the ABI call gives on the same
inputs, and reject what it documents as invalid."""
import math

import numpy as np
import pytest

import gpu_util as G
from transformer_scaled_dot_flash_amd import attn as abi
from transformer_scaled_dot_flash_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.load_library()


def _dev(seed, shape):
    return G.to_device(inputs.normal(seed, shape, "bf16"), "bf16")


def test_prefill_decode_window_match_the_abi():
    import torch
    from transformer_scaled_dot_flash_amd import ops_torch as ops
    st = torch.cuda.current_stream()
    B, H_q, H_kv, T, D = 2, 8, 2, 300, 128
    sc = float(np.float32(1 / math.sqrt(D)))
    q, k, v = _dev(981, (B, H_q, T, D)), _dev(982, (B, H_kv, T, D)), _dev(983, (B, H_kv, T, D))
    ref = torch.empty_like(q)
    abi.attn_fwd_prefill(q, k, v, ref, B, H_q, H_kv, T, T, D, True, sc, abi.ATTN_BF16, st)
    assert torch.equal(ops.prefill(q, k, v, True, sc), ref)
    abi.attn_fwd_prefill_window(q, k, v, ref, B, H_q, H_kv, T, T, D, 64, sc, abi.ATTN_BF16, st)
    assert torch.equal(ops.prefill_window(q, k, v, 64, sc), ref)
    qd = _dev(984, (B, H_q, 1, D))
    nb = abi.attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T, D, abi.ATTN_BF16, 0)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    refd = torch.empty_like(qd)
    abi.attn_fwd_decode(qd, k, v, refd, B, H_q, H_kv, 1, T, D, False, sc, abi.ATTN_BF16, 0, ws, nb, st)
    assert torch.equal(ops.decode(qd, k, v, sc), refd)
    with pytest.raises(ValueError):
        ops.prefill(q.transpose(2, 3), k, v, True, sc)  # not contiguous [B][H][T][D]


def test_varlen_and_projection_match_the_abi():
    import torch
    from transformer_scaled_dot_flash_amd import ops_torch as ops
    st = torch.cuda.current_stream()
    H_q, H_kv, D = 8, 2, 64
    lens = [100, 0, 257]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    tot = int(sum(lens))
    sc = float(np.float32(1 / math.sqrt(D)))
    q, k, v = _dev(985, (tot, H_q, D)), _dev(986, (tot, H_kv, D)), _dev(987, (tot, H_kv, D))
    ref = torch.empty_like(q)
    abi.attn_fwd_prefill_varlen(q, k, v, ref, cu, cu, 3, H_q, H_kv, D, tot, tot, 257, 257, True, 0, sc,
                                abi.ATTN_BF16, st)
    assert torch.equal(ops.prefill_varlen(q, k, v, cu, cu, 257, 257, True, sc), ref)
    with pytest.raises(TypeError):
        ops.prefill_varlen(q, k, v, cu.long(), cu, 257, 257, True, sc)
    B, T, dm = 2, 100, 256
    x, w = _dev(988, (B * T, dm)), _dev(989, ((H_q + 2 * H_kv) * D, dm))
    rq = torch.empty((B, H_q, T, D), dtype=torch.bfloat16, device="cuda")
    rk = torch.empty((B, H_kv, T, D), dtype=torch.bfloat16, device="cuda")
    rv = torch.empty_like(rk)
    abi.attn_qkv_project(x, w, rq, rk, rv, B, T, dm, H_q, H_kv, D, abi.ATTN_BF16, st)
    gq, gk, gv = ops.qkv_project(x, w, B, T, H_q, H_kv, D)
    assert torch.equal(gq, rq) and torch.equal(gk, rk) and torch.equal(gv, rv)


def test_decode_paged_matches_the_abi():
    import torch
    from transformer_scaled_dot_flash_amd import ops_torch as ops
    st = torch.cuda.current_stream()
    B, H_q, H_kv, D, ps, n_pages, max_pages = 2, 8, 2, 128, 16, 40, 12
    sc = float(np.float32(1 / math.sqrt(D)))
    q = _dev(990, (B, H_q, D))
    kp, vp = _dev(991, (n_pages, H_kv, ps, D)), _dev(992, (n_pages, H_kv, ps, D))
    table = torch.tensor(np.random.default_rng(993).permutation(n_pages)[:B * max_pages].reshape(B, max_pages),
                         dtype=torch.int32, device="cuda")
    lens = torch.tensor([150, 37], dtype=torch.int32, device="cuda")
    nb = abi.attn_fwd_decode_paged_workspace_bytes(B, H_q, H_kv, D, ps, max_pages, 0)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(q)
    abi.attn_fwd_decode_paged(q, kp, vp, ref, table, lens, B, H_q, H_kv, D, ps, n_pages, max_pages, sc,
                              abi.ATTN_BF16, 0, ws, nb, st)
    assert torch.equal(ops.decode_paged(q, kp, vp, table, lens, sc), ref)
    with pytest.raises(TypeError):
        ops.decode_paged(q, kp, vp, table.long(), lens, sc)
