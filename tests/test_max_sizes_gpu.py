"""Largest slices the C ABI accepts: one (batch, head) slice of Q and O, or of
K and V, just under 2 GiB (the kernels address a slice with 32-bit offsets
from a range-checked buffer resource, and the host rejects anything larger).

Running the oracle over eight million keys is out of reach on the CPU, so the
inputs are periodic: K and V (or Q) repeat a seeded block of 256 rows.  Each
key of the block then occurs n times with the same score, its weight is n
times larger, and the softmax-weighted mean over all keys equals the one over
a single block: the oracle on 256 keys.  Likewise an output row depends only
on its query row, so repeated query rows must give repeated output rows."""
import math

import numpy as np
import pytest

import gpu_util as G
import oracle
from transformer_scaled_dot_flash_amd import attn as abi
from transformer_scaled_dot_flash_amd import inputs

pytestmark = pytest.mark.gpu

D = 128
P = 256                                        # rows per repeated block
T_MAX = (2 ** 31 // (D * 2)) // P * P - P      # 8388352 rows: a slice of 2 GiB - 64 KiB
SCALE = float(np.float32(1.0 / math.sqrt(D)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.load_library()  # raises when the HIP library is missing: no fallback


def _f64(bits):
    return inputs.as_f64(bits, "bf16")


def _guards_intact(buf):
    """The sentinel bands around O (read back alone: O itself may be 2 GiB)."""
    s = G.SENTINEL["bf16"]
    head = buf[:G.GUARD].cpu().numpy().view(np.uint16)
    tail = buf[-G.GUARD:].cpu().numpy().view(np.uint16)
    return bool(np.all(head == s) and np.all(tail == s))


def test_prefill_kv_slice_just_under_2GiB():
    torch = G.torch_mod()
    assert T_MAX * D * 2 < 2 ** 31 and (T_MAX + P) * D * 2 >= 2 ** 31 - 2 ** 16
    T_q, H_q = 200, 2
    q = inputs.normal(901, (1, H_q, T_q, D), "bf16")
    kb = inputs.normal(902, (1, 1, P, D), "bf16")
    vb = inputs.normal(903, (1, 1, P, D), "bf16")
    want = oracle.attention(_f64(q), _f64(kb), _f64(vb), SCALE, False)
    qd = G.to_device(q, "bf16")
    kd = G.to_device(kb, "bf16").repeat(1, 1, T_MAX // P, 1)
    vd = G.to_device(vb, "bf16").repeat(1, 1, T_MAX // P, 1)
    buf, o = G.guarded_output((1, H_q, T_q, D), "bf16")
    G.note(f"attn_fwd_prefill B=1 H_q={H_q} H_kv=1 T_q={T_q} T_kv={T_MAX} D={D} causal=0 (max K/V slice)")
    abi.attn_fwd_prefill(qd, kd, vd, o, 1, H_q, 1, T_q, T_MAX, D, False, SCALE, abi.ATTN_BF16,
                         torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert _guards_intact(buf), "write outside O"
    got = G.to_f64(o, "bf16")
    del kd, vd
    torch.cuda.empty_cache()
    assert G.max_err(got, want) <= G.TOL["bf16"]


def test_prefill_q_slice_just_under_2GiB():
    torch = G.torch_mod()
    qb = inputs.normal(911, (1, 1, P, D), "bf16")
    k = inputs.normal(912, (1, 1, P, D), "bf16")
    v = inputs.normal(913, (1, 1, P, D), "bf16")
    want = oracle.attention(_f64(qb), _f64(k), _f64(v), SCALE, False)[0, 0]  # [P][D]
    qd = G.to_device(qb, "bf16").repeat(1, 1, T_MAX // P, 1)
    kd, vd = G.to_device(k, "bf16"), G.to_device(v, "bf16")
    buf, o = G.guarded_output((1, 1, T_MAX, D), "bf16")
    G.note(f"attn_fwd_prefill B=1 H_q=1 H_kv=1 T_q={T_MAX} T_kv={P} D={D} causal=0 (max Q/O slice)")
    abi.attn_fwd_prefill(qd, kd, vd, o, 1, 1, 1, T_MAX, P, D, False, SCALE, abi.ATTN_BF16,
                         torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert _guards_intact(buf), "write outside O"
    rows = np.r_[0:P, T_MAX // 2 - 3:T_MAX // 2 + 3, T_MAX - P:T_MAX]
    got = G.to_f64(o[0, 0, torch.as_tensor(rows, device="cuda")], "bf16")
    del qd, buf, o
    torch.cuda.empty_cache()
    assert G.max_err(got, want[rows % P]) <= G.TOL["bf16"]


def test_decode_kv_slice_just_under_2GiB():
    torch = G.torch_mod()
    H_q = 8
    q = inputs.normal(921, (1, H_q, 1, D), "bf16")
    kb = inputs.normal(922, (1, 1, P, D), "bf16")
    vb = inputs.normal(923, (1, 1, P, D), "bf16")
    want = oracle.attention(_f64(q), _f64(kb), _f64(vb), SCALE, False)
    qd = G.to_device(q, "bf16")
    kd = G.to_device(kb, "bf16").repeat(1, 1, T_MAX // P, 1)
    vd = G.to_device(vb, "bf16").repeat(1, 1, T_MAX // P, 1)
    buf, o = G.guarded_output((1, H_q, 1, D), "bf16")
    nbytes = abi.attn_fwd_decode_workspace_bytes(1, H_q, 1, T_MAX, D, abi.ATTN_BF16, 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    G.note(f"attn_fwd_decode B=1 H_q={H_q} H_kv=1 T_kv={T_MAX} D={D} (max K/V slice)")
    abi.attn_fwd_decode(qd, kd, vd, o, 1, H_q, 1, 1, T_MAX, D, False, SCALE, abi.ATTN_BF16, 0, ws, nbytes,
                        torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert _guards_intact(buf), "write outside O"
    got = G.to_f64(o, "bf16")
    del kd, vd
    torch.cuda.empty_cache()
    assert G.max_err(got, want) <= G.TOL["bf16"]


def test_one_row_more_is_rejected():
    """The host rejects a slice of 2 GiB or more before any launch."""
    torch = G.torch_mod()
    big = (2 ** 31) // (D * 2)  # exactly 2 GiB per slice
    q = torch.empty((1, 1, 8, D), dtype=torch.bfloat16, device="cuda")
    st = abi.attn_fwd_prefill(q, q, q, q.clone(), 1, 1, 1, 8, big, D, False, SCALE, abi.ATTN_BF16,
                              torch.cuda.current_stream(), check=False)
    assert abi.STATUS_NAMES[st] == "ATTN_ERR_INVALID_SHAPE"


def test_paged_pool_beyond_4GiB():
    """A paged cache whose pools (K and V) are 5 GiB each, with the pages of
    the sequences scattered past the 2 GiB and 4 GiB marks: page bases are
    64-bit.  Only the referenced pages are filled; the oracle sees the same
    pages compacted into a small pool."""
    import oracle.paged_fp64 as PO
    torch = G.torch_mod()
    B, H_q, H_kv, ps = 2, 8, 2, 16
    page_bytes = H_kv * ps * D * 2
    n_pages = (5 << 30) // page_bytes
    lens = [300, 1000]
    max_pages = -(-max(lens) // ps)
    rng = np.random.default_rng(931)
    marks = [0, (2 << 30) // page_bytes - 3, (4 << 30) // page_bytes - 5, n_pages - max_pages * B]
    ids = np.unique(np.concatenate([m + np.arange(max_pages * B // 2) for m in marks]))
    ids = rng.permutation(ids)[:max_pages * B]
    table = ids.reshape(B, max_pages).astype(np.int32)
    assert int(table.max()) < n_pages and int(table.max()) * page_bytes >= (4 << 30)
    q = inputs.normal(932, (B, H_q, D), "bf16")
    kp = inputs.normal(933, (ids.size, H_kv, ps, D), "bf16")  # contents of the used pages, in `ids` order
    vp = inputs.normal(934, (ids.size, H_kv, ps, D), "bf16")
    k_pool = torch.empty((n_pages, H_kv, ps, D), dtype=torch.bfloat16, device="cuda")
    v_pool = torch.empty_like(k_pool)
    where = torch.as_tensor(ids, dtype=torch.int64, device="cuda")
    k_pool[where] = G.to_device(kp, "bf16")
    v_pool[where] = G.to_device(vp, "bf16")
    qd = G.to_device(q, "bf16")
    td = torch.from_numpy(table).cuda()
    ld = torch.as_tensor(lens, dtype=torch.int32, device="cuda")
    buf, o = G.guarded_output((B, H_q, D), "bf16")
    nbytes = abi.attn_fwd_decode_paged_workspace_bytes(B, H_q, H_kv, D, ps, max_pages, 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    G.note(f"attn_fwd_decode_paged B={B} H_q={H_q} H_kv={H_kv} D={D} page={ps} pages={n_pages} (5 GiB pools)")
    abi.attn_fwd_decode_paged(qd, k_pool, v_pool, o, td, ld, B, H_q, H_kv, D, ps, n_pages, max_pages, SCALE,
                              abi.ATTN_BF16, 0, ws, nbytes, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert _guards_intact(buf), "write outside O"
    got = G.to_f64(o, "bf16")
    del k_pool, v_pool
    torch.cuda.empty_cache()
    compact = np.arange(ids.size, dtype=np.int32).reshape(B, max_pages)  # table over the compacted pool
    want = PO.decode_paged(_f64(q), _f64(kp), _f64(vp), compact, np.asarray(lens, np.int32), SCALE)
    assert G.max_err(got, want) <= G.TOL["bf16"]


def _run_varlen(qd, kd, vd, cu_q, cu_k, H_q, H_kv, causal):
    torch = G.torch_mod()
    lq, lk = np.diff(cu_q), np.diff(cu_k)
    total_q, total_k = int(cu_q[-1]), int(cu_k[-1])
    cq = torch.as_tensor(np.asarray(cu_q, np.int32), device="cuda")
    ck = torch.as_tensor(np.asarray(cu_k, np.int32), device="cuda")
    buf, o = G.guarded_output((total_q, H_q, D), "bf16")
    G.note(f"attn_fwd_prefill_varlen B={len(lq)} H_q={H_q} H_kv={H_kv} D={D} total_q={total_q} "
           f"total_k={total_k} causal={int(causal)} (packed buffers over 4 GiB)")
    abi.attn_fwd_prefill_varlen(qd, kd, vd, o, cq, ck, len(lq), H_q, H_kv, D, total_q, total_k,
                                int(lq.max()), int(lk.max()), causal, 0, SCALE, abi.ATTN_BF16,
                                torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert _guards_intact(buf), "write outside O"
    return buf, o


def test_varlen_packed_q_beyond_4GiB():
    """Three sequences of 199,936 query rows each (Q and O 4.6 GiB, the last
    sequence starting past 4 GiB) against 256 keys each; every sequence's
    queries repeat a seeded 256-row block, so its output rows repeat the
    oracle's rows for that block."""
    torch = G.torch_mod()
    H_q, H_kv, L = 32, 8, 781 * P
    assert (L + 256) * H_q * D * 2 < 2 ** 31 and 3 * L * H_q * D * 2 > (4 << 30)
    cu_q = np.array([0, L, 2 * L, 3 * L])
    cu_k = np.array([0, P, 2 * P, 3 * P])
    qb = inputs.normal(941, (3, P, H_q, D), "bf16")
    k = inputs.normal(942, (3 * P, H_kv, D), "bf16")
    v = inputs.normal(943, (3 * P, H_kv, D), "bf16")
    qd = G.to_device(qb, "bf16").repeat(1, L // P, 1, 1).reshape(3 * L, H_q, D)
    buf, o = _run_varlen(qd, G.to_device(k, "bf16"), G.to_device(v, "bf16"), cu_q, cu_k, H_q, H_kv, False)
    rows = np.r_[0:8, L - 8:L + 8, 2 * L:2 * L + 8, 3 * L - P:3 * L]
    got = G.to_f64(o[torch.as_tensor(rows, device="cuda")], "bf16")
    del qd, buf, o
    torch.cuda.empty_cache()
    for s in range(3):
        want = oracle.attention_varlen(_f64(qb[s]), _f64(k[s * P:(s + 1) * P]), _f64(v[s * P:(s + 1) * P]),
                                       [0, P], [0, P], SCALE, False)
        sel = (rows >= s * L) & (rows < (s + 1) * L)
        assert G.max_err(got[sel], want[(rows[sel] - s * L) % P]) <= G.TOL["bf16"]


def test_varlen_packed_kv_beyond_4GiB():
    """Three sequences of 100 queries against 819,200 keys each (K and V
    4.7 GiB, the last sequence's keys past 4 GiB); every sequence's keys and
    values repeat a seeded 256-key block, so its output equals the oracle's
    over that block."""
    torch = G.torch_mod()
    H_q, H_kv, Lq, L = 8, 8, 100, 3200 * P
    assert (L + 64) * H_kv * D * 2 < 2 ** 31 and 3 * L * H_kv * D * 2 > (4 << 30)
    cu_q = np.array([0, Lq, 2 * Lq, 3 * Lq])
    cu_k = np.array([0, L, 2 * L, 3 * L])
    q = inputs.normal(951, (3 * Lq, H_q, D), "bf16")
    kb = inputs.normal(952, (3, P, H_kv, D), "bf16")
    vb = inputs.normal(953, (3, P, H_kv, D), "bf16")
    kd = G.to_device(kb, "bf16").repeat(1, L // P, 1, 1).reshape(3 * L, H_kv, D)
    vd = G.to_device(vb, "bf16").repeat(1, L // P, 1, 1).reshape(3 * L, H_kv, D)
    buf, o = _run_varlen(G.to_device(q, "bf16"), kd, vd, cu_q, cu_k, H_q, H_kv, False)
    got = G.to_f64(o, "bf16")
    del kd, vd, buf, o
    torch.cuda.empty_cache()
    for s in range(3):
        want = oracle.attention_varlen(_f64(q[s * Lq:(s + 1) * Lq]), _f64(kb[s]), _f64(vb[s]),
                                       [0, Lq], [0, P], SCALE, False)
        assert G.max_err(got[s * Lq:(s + 1) * Lq], want) <= G.TOL["bf16"]


def test_qkv_projection_tensors_just_under_2GiB():
    """X and Q of the fused projection each just under 2 GiB (the host limit:
    every tensor is addressed with 32-bit offsets), B = 3 sequences of 87,296
    tokens; X repeats a seeded 256-token block, so output token m equals the
    oracle's projection of block row m mod 256.  Bound as for the other
    projection tests: |dY| <= 1e-3 + 2^-8 |Y|."""
    import oracle.qkv_fp64 as QP
    torch = G.torch_mod()
    B, T, dm, H_q, H_kv = 3, 341 * P, 4096, 32, 8
    M, N = B * T, (H_q + 2 * H_kv) * D
    assert M * dm * 2 < 2 ** 31 and M * H_q * D * 2 < 2 ** 31 and (M + P) * dm * 2 >= 2 ** 31
    xb = inputs.normal(971, (P, dm), "bf16")
    w32 = inputs.bf16_bits_to_f32(inputs.normal(972, (N, dm), "bf16")) / np.float32(np.sqrt(dm))
    w = inputs.f32_to_bf16_bits(w32)
    xd = G.to_device(xb, "bf16").repeat(M // P, 1)
    bq, qo = G.guarded_output((B, H_q, T, D), "bf16")
    bk, ko = G.guarded_output((B, H_kv, T, D), "bf16")
    bv, vo = G.guarded_output((B, H_kv, T, D), "bf16")
    G.note(f"attn_qkv_project B={B} T={T} d_model={dm} H_q={H_q} H_kv={H_kv} D={D} (X, Q near 2 GiB)")
    abi.attn_qkv_project(xd, G.to_device(w, "bf16"), qo, ko, vo, B, T, dm, H_q, H_kv, D, abi.ATTN_BF16,
                         torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert all(_guards_intact(b) for b in (bq, bk, bv)), "write outside an output"
    y = QP.project(_f64(xb), _f64(w))  # [P][N]: the block's projection
    qn, kn = H_q * D, H_kv * D
    for b, t in [(0, 0), (0, 255), (1, 5), (1, T - 1), (2, 7), (2, T // 2 + 3), (2, T - 1)]:
        want = y[(b * T + t) % P]
        for got, ref in ((qo[b, :, t], want[:qn]), (ko[b, :, t], want[qn:qn + kn]), (vo[b, :, t], want[qn + kn:])):
            g = G.to_f64(got.reshape(-1), "bf16")
            assert np.all(np.abs(g - ref) <= 1e-3 + np.abs(ref) * 2.0 ** -8), f"token ({b}, {t})"
    del xd, bq, qo, bk, ko, bv, vo
    torch.cuda.empty_cache()
