"""GPU parity of the paged-KV decode (attn_fwd_decode_paged) against the
paged oracle, on seeded inputs laid out in shuffled page pools.

Bar: max |O_gpu - O_oracle| <= 1.5e-2 (bf16) over every element; no write
outside O (sentinel guard bands); no element of O left unwritten.  Also: the
paged kernel reproduces the contiguous decode kernel bit for bit when the
pages hold the same keys, and the documented readings for empty sequences and
out-of-pool block ids."""
import zlib

import numpy as np
import pytest

import gpu_util as G
import oracle.paged_fp64 as P
from transformer_scaled_dot_flash_amd import attn as abi
from transformer_scaled_dot_flash_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.load_library()


def _seed(*case):
    return zlib.crc32(repr(case).encode())


def make_case(B, H_q, H_kv, D, ps, lens, extra_pages=3, seed=0):
    """Seeded q and pools; each sequence gets ceil(len / ps) pages in a shuffled
    pool (unused rows and pages hold other seeded values)."""
    s = _seed(B, H_q, H_kv, D, ps, tuple(lens), seed)
    max_pages = max(1, max(-(-L // ps) for L in lens))
    n_pages = B * max_pages + extra_pages
    q = inputs.normal(s + 1, (B, H_q, D), "bf16")
    kp = inputs.normal(s + 2, (n_pages, H_kv, ps, D), "bf16")
    vp = inputs.normal(s + 3, (n_pages, H_kv, ps, D), "bf16")
    perm = np.random.default_rng(s).permutation(n_pages)
    table = perm[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    return q, kp, vp, table, np.asarray(lens, np.int32)


def run_paged(q, kp, vp, table, lens, scale, num_splits=0):
    torch = G.torch_mod()
    B, H_q, D = q.shape
    n_pages, H_kv, ps, _ = kp.shape
    max_pages = table.shape[1]
    qd, kd, vd = (G.to_device(x, "bf16") for x in (q, kp, vp))
    td = torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda()
    ld = torch.from_numpy(np.ascontiguousarray(lens, np.int32)).cuda()
    buf, o = G.guarded_output((B, H_q, D), "bf16")
    nbytes = abi.attn_fwd_decode_paged_workspace_bytes(B, H_q, H_kv, D, ps, max_pages, num_splits)
    ws = torch.full((max(nbytes, 16) // 4,), -1, dtype=torch.int32, device="cuda")
    G.note(f"attn_fwd_decode_paged B={B} H_q={H_q} H_kv={H_kv} D={D} page={ps} pages={n_pages} "
           f"max_pages={max_pages} splits={num_splits} lens={list(lens)[:8]}")
    abi.attn_fwd_decode_paged(qd, kd, vd, o, td, ld, B, H_q, H_kv, D, ps, n_pages, max_pages, scale,
                              abi.ATTN_BF16, num_splits, ws, nbytes, torch.cuda.current_stream())
    torch.cuda.synchronize()
    G.check_guards(buf, "bf16", "paged decode")
    return G.to_f64(o, "bf16")


def oracle_paged(q, kp, vp, table, lens, scale):
    return P.decode_paged(inputs.as_f64(q, "bf16"), inputs.as_f64(kp, "bf16"),
                          inputs.as_f64(vp, "bf16"), table, lens, scale)


CASES = [
    # B, H_q, H_kv, D, page_size, seq_lens, splits
    (1, 1, 1, 64, 16, [1], 0),
    (3, 8, 2, 128, 16, [1, 15, 16], 0),
    (3, 8, 2, 128, 16, [17, 31, 32], 0),
    (4, 4, 4, 64, 16, [33, 100, 257, 64], 0),
    (2, 32, 8, 128, 16, [1000, 4096], 0),
    (2, 32, 8, 128, 32, [777, 1], 0),
    (2, 8, 1, 64, 64, [300, 129], 0),        # MQA
    (2, 40, 8, 128, 16, [513, 96], 0),       # G = 5
    (1, 64, 1, 128, 16, [200], 0),           # 64 q heads on one kv head: two MFMA column blocks
    (3, 8, 2, 128, 16, [700, 5, 1024], 1),
    (3, 8, 2, 128, 16, [700, 5, 1024], 3),
    (3, 8, 2, 128, 16, [700, 5, 1024], 8),
    (2, 16, 4, 64, 128, [2048, 1500], 16),
    (1, 4, 2, 128, 1024, [3000], 2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}H{c[1]}/{c[2]}D{c[3]}p{c[4]}s{c[6]}")
def test_paged_matches_oracle(case):
    B, H_q, H_kv, D, ps, lens, splits = case
    q, kp, vp, table, L = make_case(B, H_q, H_kv, D, ps, lens)
    scale = 1.0 / np.sqrt(D)
    got = run_paged(q, kp, vp, table, L, scale, splits)
    want = oracle_paged(q, kp, vp, table, L, scale)
    err = G.max_err(got, want)
    print(f"paged {case}: max|dO| = {err:.3e}")
    assert err <= G.TOL["bf16"]


def test_paged_equals_contiguous_decode_bitwise():
    # Pages holding each sequence's keys in order reproduce the contiguous
    # layout; with the same split plan the two kernels do identical work.
    B, H_q, H_kv, T, D, ps = 3, 16, 4, 1024, 128, 16
    s = _seed("contig", B, H_q, H_kv, T, D)
    q = inputs.normal(s + 1, (B, H_q, 1, D), "bf16")
    k = inputs.normal(s + 2, (B, H_kv, T, D), "bf16")
    v = inputs.normal(s + 3, (B, H_kv, T, D), "bf16")
    per = T // ps
    rng = np.random.default_rng(s)
    perm = rng.permutation(B * per)
    kp = np.empty((B * per, H_kv, ps, D), np.uint16)
    vp = np.empty_like(kp)
    table = np.empty((B, per), np.int32)
    for b in range(B):
        for p in range(per):
            table[b, p] = perm[b * per + p]
            kp[perm[b * per + p]] = k[b, :, p * ps:(p + 1) * ps]
            vp[perm[b * per + p]] = v[b, :, p * ps:(p + 1) * ps]
    for splits in (1, 4):
        a = G.decode(q, k, v, 0.088, "bf16", splits)[:, :, 0]
        b = run_paged(q[:, :, 0], kp, vp, table, np.full(B, T, np.int32), 0.088, splits)
        assert np.array_equal(a, b), f"splits={splits}: paged and contiguous decode differ"


def test_paged_empty_sequence_gives_zero():
    q, kp, vp, table, L = make_case(3, 8, 2, 128, 16, [0, 40, 0])
    for splits in (0, 4):
        got = run_paged(q, kp, vp, table, L, 0.1, splits)
        assert np.all(got[0] == 0) and np.all(got[2] == 0)
        want = oracle_paged(q, kp, vp, table, L, 0.1)
        assert G.max_err(got, want) <= G.TOL["bf16"]


def test_paged_out_of_pool_block_reads_zeros():
    q, kp, vp, table, L = make_case(2, 8, 2, 64, 16, [64, 48])
    table = table.copy()
    table[0, 1] = kp.shape[0] + 7    # past the pool
    table[1, 0] = -3                 # negative
    got = run_paged(q, kp, vp, table, L, 0.2)
    want = oracle_paged(q, kp, vp, table, L, 0.2)
    assert G.max_err(got, want) <= G.TOL["bf16"]


def test_paged_length_clamped_to_table_capacity():
    q, kp, vp, table, L = make_case(2, 4, 1, 64, 16, [32, 20])
    long = np.array([10_000, 20], np.int32)
    a = run_paged(q, kp, vp, table, long, 0.2)
    b = run_paged(q, kp, vp, table, np.array([32, 20], np.int32), 0.2)
    assert np.array_equal(a, b)


def test_paged_deterministic():
    q, kp, vp, table, L = make_case(2, 32, 8, 128, 16, [3000, 77])
    a = run_paged(q, kp, vp, table, L, 0.09, 8)
    b = run_paged(q, kp, vp, table, L, 0.09, 8)
    assert np.array_equal(a, b)
