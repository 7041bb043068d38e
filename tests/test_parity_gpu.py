"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle,
element by element on the same seeded inputs.

Bar: max |O_gpu - O_oracle| <= 1e-5 for fp32 tensors and <= 1.5e-2 for bf16
tensors, over every compared element.  Where the bf16 output format itself
cannot meet 1.5e-2 (|O| >= 4, half an ulp is 1/64; only at scales well above
1/sqrt(D)), an element is judged by its own arithmetic bound instead
(gpu_util.check_bf16_prefill); the workloads must meet the plain bar.  Also
checked on every call: no write outside O (sentinel guard bands) and no
element of O left unwritten (O starts as NaN)."""
import math
import zlib

import numpy as np
import pytest

import gpu_util as G
import oracle
from transformer_scaled_dot_flash_amd import attn as abi
from transformer_scaled_dot_flash_amd import inputs
from transformer_scaled_dot_flash_amd.workloads import BY_ORDINAL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.load_library()  # raises when the HIP library is missing: no fallback


def gen(seed, shape, dtype):
    return inputs.normal(seed, shape, dtype)


def f64(x, dtype):
    return inputs.as_f64(x, dtype)


# --- the five workloads ----------------------------------------------------------
@pytest.mark.parametrize("ordinal", [1, 2, 3, 4, 5])
def test_workload_parity(ordinal):
    """Every element of every workload's output against the oracle (the
    T=8192 GQA prefill too: 32 heads x 8192 rows, ~15 s of host time)."""
    w = BY_ORDINAL[ordinal]
    q, k, v = w.make_inputs()
    Q, K, V = f64(q, w.dtype), f64(k, w.dtype), f64(v, w.dtype)
    if w.kind == "decode":
        got = G.decode(q, k, v, w.scale, w.dtype)
    else:
        got = G.prefill(q, k, v, w.causal, w.scale, w.dtype)
    want = oracle.attention(Q, K, V, w.scale, w.causal)
    if ordinal == 4:
        # causal row 0 sees only key 0: O equals V[0] bit for bit
        assert np.array_equal(got[:, :, 0], V[:, np.arange(w.H_q) // (w.H_q // w.H_kv), 0])
    rel = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    if w.dtype == "bf16":
        err, floor, n_bound = G.check_bf16_prefill(got, want, Q, K, V, w.scale, w.causal, what=w.name)
        print(f"{w.name}: max|dO| = {err:.3e}, bf16 floor {floor:.3e}, rel. Frobenius {rel:.3e}, "
              f"elements judged by the arithmetic bound: {n_bound}")
        assert n_bound == 0 and err <= G.TOL["bf16"], f"{w.name}: max|dO| {err:.3e}"
    else:
        err = G.max_err(got, want)
        print(f"{w.name}: max|dO| = {err:.3e}, rel. Frobenius {rel:.3e}")
        assert err <= G.TOL[w.dtype], f"{w.name}: max|dO| {err:.3e} > {G.TOL[w.dtype]}"


# Shapes and seeds (found by a CPU scan) whose exact output has rows with
# |O| >= 4 at scale 4/sqrt(D): there half a bf16 ulp is 1/64, so even the
# correctly rounded exact result misses 1.5e-2 and the per-element
# arithmetic bound judges those elements.
FLOOR_CASES = [(185, 1, 8, 2, 128, 128, False), (334, 1, 8, 1, 128, 64, True)]


@pytest.mark.parametrize("case", FLOOR_CASES, ids=lambda c: "-".join(map(str, c)))
def test_bf16_output_floor_cases(case):
    seed, B, H_q, H_kv, T, D, causal = case
    q = gen(seed, (B, H_q, T, D), "bf16")
    k = gen(seed + 1, (B, H_kv, T, D), "bf16")
    v = gen(seed + 2, (B, H_kv, T, D), "bf16")
    Q, K, V = f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16")
    scale = float(np.float32(4.0 / math.sqrt(D)))
    want = oracle.attention(Q, K, V, scale, causal)
    assert G.bf16_floor(want) > G.TOL["bf16"]
    got = G.prefill(q, k, v, causal, scale, "bf16")
    err, floor, n_bound = G.check_bf16_prefill(got, want, Q, K, V, scale, causal, what=str(case))
    print(f"{case}: max|dO| = {err:.4e}, bf16 floor {floor:.4e}, judged by the bound: {n_bound}")
    assert err <= 2 * floor


# --- ragged and edge shapes ----------------------------------------------------------
PREFILL_CASES = [
    # B, H_q, H_kv, T_q, T_kv, D, causal, dtype
    (1, 1, 1, 1, 1, 64, True, "bf16"),
    (1, 1, 1, 1, 1, 128, False, "bf16"),
    (1, 2, 1, 7, 7, 64, True, "bf16"),
    (2, 4, 2, 100, 100, 128, True, "bf16"),
    (1, 3, 3, 129, 129, 64, True, "bf16"),
    (1, 2, 2, 257, 257, 128, False, "bf16"),
    (1, 8, 1, 300, 300, 128, True, "bf16"),      # MQA
    (2, 6, 2, 191, 191, 64, False, "bf16"),
    (1, 4, 4, 1000, 1000, 64, True, "bf16"),
    (1, 4, 2, 384, 384, 128, True, "bf16"),
    (1, 2, 1, 65, 300, 128, True, "bf16"),       # chunked causal: T_q < T_kv
    (1, 2, 2, 33, 1000, 64, True, "bf16"),
    (1, 2, 2, 50, 77, 128, False, "bf16"),       # non-causal T_q != T_kv
    (1, 2, 2, 300, 40, 64, False, "bf16"),       # more queries than keys
    (8, 16, 8, 64, 64, 128, True, "bf16"),       # 64 kv units: XCD placement path
    (2, 32, 8, 1100, 1100, 64, True, "bf16"),    # grid too large for the key split: 4-wave shape
    (1, 32, 8, 1100, 1100, 128, True, "bf16"),   # the same at D = 128
    (1, 8, 2, 1000, 1000, 64, True, "bf16"),     # key split, odd number of key tiles per group
    (1, 4, 4, 130, 2000, 128, True, "bf16"),     # key split, chunk of queries at the end of the keys
    (1, 2, 1, 200, 200, 128, False, "bf16"),     # key split, non-causal
    (1, 1, 1, 128, 128, 64, False, "f32"),
    (1, 1, 1, 1, 1, 64, True, "f32"),
    (2, 4, 2, 100, 100, 128, True, "f32"),
    (1, 6, 3, 77, 130, 64, True, "f32"),
    (1, 4, 1, 33, 33, 128, False, "f32"),
    # fp32 above 2^24 (row, key) pairs: the 64-rows-per-workgroup kernel instead of one wave per row
    (1, 4, 2, 2100, 2100, 64, True, "f32"),
    (1, 2, 1, 1500, 6000, 128, False, "f32"),
    (1, 1, 1, 4096, 4096, 64, True, "f32"),       # exactly 2^24 pairs: the last size on one wave per row
    (1, 1, 1, 4096, 4097, 64, True, "f32"),       # one key more: the 64-row kernel
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "-".join(map(str, c)))
def test_prefill_ragged(case):
    B, H_q, H_kv, T_q, T_kv, D, causal, dtype = case
    seed = 100 + zlib.crc32(repr(case).encode()) % 1000
    q = gen(seed, (B, H_q, T_q, D), dtype)
    k = gen(seed + 1, (B, H_kv, T_kv, D), dtype)
    v = gen(seed + 2, (B, H_kv, T_kv, D), dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    got = G.prefill(q, k, v, causal, scale, dtype)
    want = oracle.attention(f64(q, dtype), f64(k, dtype), f64(v, dtype), scale, causal)
    err = G.max_err(got, want)
    assert err <= G.TOL[dtype], f"{case}: max|dO| {err:.3e}"


DECODE_CASES = [
    # B, H_q, H_kv, T_kv, D, dtype, splits
    (4, 32, 8, 1000, 128, "bf16", 1),
    (4, 32, 8, 1000, 128, "bf16", 2),
    (4, 32, 8, 1000, 128, "bf16", 8),
    (4, 32, 8, 1000, 128, "bf16", 64),
    (2, 8, 8, 1, 128, "bf16", 0),
    (2, 8, 2, 31, 64, "bf16", 0),
    (2, 8, 2, 33, 64, "bf16", 3),
    (3, 64, 1, 4097, 128, "bf16", 0),   # 64 q heads per kv head: two head blocks
    (1, 40, 5, 777, 64, "bf16", 5),
    (2, 16, 16, 300, 128, "bf16", 0),   # MHA decode
    (1, 8, 2, 6000, 64, "bf16", 150),   # more than 64 splits: several rounds per combine lane
    (1, 16, 4, 20000, 64, "bf16", 0),   # default plan at D = 64 with few groups: 125 splits
    (2, 8, 2, 300, 128, "f32", 0),
    (1, 4, 1, 65, 64, "f32", 0),
    (2, 64, 1, 140000, 64, "f32", 0),   # above 2^24 (row, key) pairs: the 64-row fp32 kernel
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_ragged(case):
    B, H_q, H_kv, T_kv, D, dtype, splits = case
    seed = 300 + zlib.crc32(repr(case).encode()) % 1000
    q = gen(seed, (B, H_q, 1, D), dtype)
    k = gen(seed + 1, (B, H_kv, T_kv, D), dtype)
    v = gen(seed + 2, (B, H_kv, T_kv, D), dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    got = G.decode(q, k, v, scale, dtype, splits)
    want = oracle.attention(f64(q, dtype), f64(k, dtype), f64(v, dtype), scale, False)
    err = G.max_err(got, want)
    assert err <= G.TOL[dtype], f"{case}: max|dO| {err:.3e}"


def test_decode_split_count_changes_only_rounding():
    B, H_q, H_kv, T_kv, D = 2, 8, 2, 2048, 128
    q = gen(501, (B, H_q, 1, D), "bf16")
    k = gen(502, (B, H_kv, T_kv, D), "bf16")
    v = gen(503, (B, H_kv, T_kv, D), "bf16")
    outs = [G.decode(q, k, v, 0.088, "bf16", n) for n in (1, 2, 8, 64)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 2 * 2.0 ** -9 * max(1.0, np.max(np.abs(outs[0])))


# --- facts that pin single values exactly ---------------------------------------------
@pytest.mark.parametrize("D", [64, 128])
def test_causal_row0_is_v0_bitwise(D):
    B, H_q, H_kv, T = 2, 8, 2, 300
    q = gen(601, (B, H_q, T, D), "bf16")
    k = gen(602, (B, H_kv, T, D), "bf16")
    v = gen(603, (B, H_kv, T, D), "bf16")
    got = G.prefill(q, k, v, True, 0.125, "bf16")
    V = f64(v, "bf16")
    for h in range(H_q):
        assert np.array_equal(got[:, h, 0], V[:, h // (H_q // H_kv), 0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_query_gives_mean_of_visible_values(dtype):
    B, H_q, H_kv, T, D = 1, 4, 2, 200, 64
    q = np.zeros((B, H_q, T, D), np.uint16 if dtype == "bf16" else np.float32)
    k = gen(611, (B, H_kv, T, D), dtype)
    rng = np.random.default_rng(7)
    vv = rng.integers(-8, 9, (B, H_kv, T, D)).astype(np.float32)  # exact in bf16
    v = inputs.f32_to_bf16_bits(vv) if dtype == "bf16" else vv
    got = G.prefill(q, k, v, True, 0.125, dtype)
    csum = np.cumsum(vv.astype(np.float64), axis=2)
    want = csum / np.arange(1, T + 1)[None, None, :, None]
    want = np.repeat(want, H_q // H_kv, axis=1)
    floor = G.bf16_floor(want) if dtype == "bf16" else 0.0
    assert G.max_err(got, want) <= floor + 1e-6


def test_gqa_head_mapping_exact():
    B, H_q, H_kv, T, D = 1, 8, 4, 96, 128
    q = gen(621, (B, H_q, T, D), "bf16")
    k = gen(622, (B, H_kv, T, D), "bf16")
    vv = np.zeros((B, H_kv, T, D), np.float32)
    for g in range(H_kv):
        vv[:, g] = g + 1.0
    v = inputs.f32_to_bf16_bits(vv)
    for causal in (False, True):
        got = G.prefill(q, k, v, causal, 0.088, "bf16")
        for h in range(H_q):
            assert np.all(got[:, h] == h // 2 + 1.0), f"q head {h} read the wrong kv head"


def test_decode_structural_facts():
    B, H_q, H_kv, T, D = 2, 32, 8, 4096, 128
    # V constant: O is that constant
    q = gen(631, (B, H_q, 1, D), "bf16")
    k = gen(632, (B, H_kv, T, D), "bf16")
    v = inputs.f32_to_bf16_bits(np.full((B, H_kv, T, D), 0.75, np.float32))
    assert np.all(G.decode(q, k, v, 0.088, "bf16") == 0.75)
    # Q = 0 and V[j, d] = 1 iff key j lies in chunk d (32 keys per chunk): O = 1/128 exactly
    q0 = np.zeros((B, H_q, 1, D), np.uint16)
    vv = np.zeros((B, H_kv, T, D), np.float32)
    for d in range(D):
        vv[:, :, 32 * d:32 * (d + 1), d] = 1.0
    got = G.decode(q0, k, inputs.f32_to_bf16_bits(vv), 0.088, "bf16")
    assert np.all(got == 1.0 / 128.0)
    # one dominant key: O equals its value row to bf16 rounding
    kk = f64(k, "bf16").astype(np.float32)
    qq = np.zeros((B, H_q, 1, D), np.float32)
    jstar = 1234
    for b in range(B):
        for h in range(H_q):
            qq[b, h, 0] = kk[b, h // 4, jstar] * 4.0
    vr = gen(633, (B, H_kv, T, D), "bf16")
    got = G.decode(inputs.f32_to_bf16_bits(qq), k, vr, 0.088, "bf16")
    want = oracle.attention(f64(inputs.f32_to_bf16_bits(qq), "bf16"), f64(k, "bf16"), f64(vr, "bf16"),
                            0.088, False)
    assert G.max_err(got, want) <= G.TOL["bf16"]
    # jointly permuting keys and values leaves O unchanged (to rounding)
    perm = np.random.default_rng(3).permutation(T)
    base = G.decode(q, k, vr, 0.088, "bf16")
    permd = G.decode(q, k[:, :, perm], vr[:, :, perm], 0.088, "bf16")
    assert np.max(np.abs(base - permd)) <= 2 * 2.0 ** -9 * max(1.0, np.max(np.abs(base)))


def test_large_logits_stay_finite():
    B, H_q, H_kv, T, D = 1, 4, 2, 256, 128
    q = gen(641, (B, H_q, T, D), "bf16")
    k = gen(642, (B, H_kv, T, D), "bf16")
    v = gen(643, (B, H_kv, T, D), "bf16")
    scale = float(np.float32(100.0 / math.sqrt(D)))
    for causal in (False, True):
        got = G.prefill(q, k, v, causal, scale, "bf16")
        want = oracle.attention(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), scale, causal)
        assert G.max_err(got, want) <= G.TOL["bf16"]


def _ramped_keys(k, direction):
    """K with key j's row scaled by 1 + 3j/T (direction +1: scores grow along
    the keys, so running row maxima keep jumping) or by 4 - 3j/T (direction
    -1: early keys dominate and later weights sit far below the base);
    rounded back to bf16."""
    K = f64(k, "bf16")
    T = K.shape[2]
    j = np.arange(T, dtype=np.float64) / T
    ramp = 1.0 + 3.0 * j if direction > 0 else 4.0 - 3.0 * j
    return inputs.f32_to_bf16_bits((K * ramp[None, None, :, None]).astype(np.float32))


@pytest.mark.parametrize("direction", [1, -1])
@pytest.mark.parametrize("B,H_q,H_kv,T,D,causal,rows", [
    (1, 4, 2, 1100, 128, True, None),
    (2, 4, 4, 700, 64, False, None),
    (1, 32, 8, 4100, 128, True, list(range(0, 40)) + list(range(2000, 2040)) + list(range(4060, 4100))),
])
def test_exponent_base_moves_on_later_tiles(direction, B, H_q, H_kv, T, D, causal, rows):
    """The prefill kernels keep a row's exponent base until the weights grow
    too large and then move it to the exact row maximum; growing scores make
    that happen on many later tiles (both launch shapes: the last case uses
    the 8-wave one)."""
    seed = 671 + T + D + direction
    q = gen(seed, (B, H_q, T, D), "bf16")
    k = _ramped_keys(gen(seed + 1, (B, H_kv, T, D), "bf16"), direction)
    v = gen(seed + 2, (B, H_kv, T, D), "bf16")
    scale = float(np.float32(1.0 / math.sqrt(D)))
    got = G.prefill(q, k, v, causal, scale, "bf16")
    assert np.all(np.isfinite(got))
    want = oracle.attention(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), scale, causal, rows=rows)
    if rows is not None:
        got = got[:, :, rows]
    err = G.max_err(got, want)
    assert err <= G.TOL["bf16"], f"max|dO| {err:.3e}"


# --- the check has teeth: the pages' pitfalls must fail it -----------------------------
def test_negative_controls_exceed_tolerance():
    w = BY_ORDINAL[2]
    q, k, v = w.make_inputs()
    Q, K, V = f64(q, w.dtype), f64(k, w.dtype), f64(v, w.dtype)
    got = G.prefill(q, k, v, True, w.scale, w.dtype)
    tol = G.TOL[w.dtype]
    assert G.max_err(got, oracle.attention(Q, K, V, w.scale, True)) <= tol
    wrong = {
        "mask direction (non-causal)": oracle.attention(Q, K, V, w.scale, False),
        "scale 1/D": oracle.attention(Q, K, V, 1.0 / w.D, True),
        "K and V swapped": oracle.attention(Q, V, K, w.scale, True),
    }
    for name, ref in wrong.items():
        assert G.max_err(got, ref) > tol, f"negative control '{name}' passed the parity check"


# --- runtime behaviour ------------------------------------------------------------------
def test_deterministic_bitwise():
    w = BY_ORDINAL[3]
    q, k, v = w.make_inputs()
    a = G.prefill(q, k, v, True, w.scale, w.dtype)
    b = G.prefill(q, k, v, True, w.scale, w.dtype)
    assert np.array_equal(a, b)
    w5 = BY_ORDINAL[5]
    q, k, v = (x[:8] for x in w5.make_inputs())
    assert np.array_equal(G.decode(q, k, v, w5.scale, "bf16"), G.decode(q, k, v, w5.scale, "bf16"))


def test_empty_problems_are_noops():
    import torch
    e = torch.empty((0, 4, 16, 64), dtype=torch.bfloat16, device="cuda")
    kk = torch.empty((0, 4, 16, 64), dtype=torch.bfloat16, device="cuda")
    assert abi.attn_fwd_prefill(e, kk, kk, e, 0, 4, 4, 16, 16, 64, True, 0.125, abi.ATTN_BF16,
                                torch.cuda.current_stream()) == 0
    q = torch.zeros((1, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 4, 16, 64), dtype=torch.bfloat16, device="cuda")
    assert abi.attn_fwd_prefill(q, k, k, q, 1, 4, 4, 0, 16, 64, True, 0.125, abi.ATTN_BF16,
                                torch.cuda.current_stream()) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("D,causal,H_q,H_kv,B", [(128, True, 64, 8, 1), (64, False, 32, 32, 2),
                                                  (64, True, 36, 3, 1)])  # 3 kv units: no XCD grouping
def test_large_problem_configuration_sampled(D, causal, H_q, H_kv, B):
    """Shapes big enough for the 8-wave prefill configuration (T >= 4096 and
    at least 512 workgroups of 256 rows), ragged T."""
    T = 4100
    q = gen(661 + D, (B, H_q, T, D), "bf16")
    k = gen(662 + D, (B, H_kv, T, D), "bf16")
    v = gen(663 + D, (B, H_kv, T, D), "bf16")
    scale = float(np.float32(1.0 / math.sqrt(D)))
    got = G.prefill(q, k, v, causal, scale, "bf16")
    rows = list(range(0, 130)) + list(range(2040, 2070)) + list(range(4050, 4100))
    want = oracle.attention(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), scale, causal, rows=rows)
    assert G.max_err(got[:, :, rows], want) <= G.TOL["bf16"]


def test_long_sequence_sampled():
    B, H, T, D = 1, 1, 32768, 128
    q = gen(651, (B, H, T, D), "bf16")
    k = gen(652, (B, H, T, D), "bf16")
    v = gen(653, (B, H, T, D), "bf16")
    got = G.prefill(q, k, v, True, 0.088, "bf16")
    rows = [0, 1, 127, 128, 16383, 16384, 32640, 32767]
    want = oracle.attention(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), 0.088, True, rows=rows)
    assert G.max_err(got[:, :, rows], want) <= G.TOL["bf16"]


def test_library_loaded_before_torch_in_a_fresh_process():
    """Loading the library before torch must not leave the process with two
    HIP runtimes (torch bundles its own): a prefill in a fresh interpreter
    whose first act is load_library() matches the oracle."""
    import subprocess
    import sys
    from pathlib import Path
    root = Path(__file__).resolve().parent.parent
    code = (
        "import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "from transformer_scaled_dot_flash_amd import attn as abi\n"
        "abi.load_library()\n"
        "import numpy as np, gpu_util as G, oracle\n"
        "from transformer_scaled_dot_flash_amd import inputs\n"
        "q = inputs.normal(961, (1, 2, 70, 64), 'bf16'); k = inputs.normal(962, (1, 1, 90, 64), 'bf16')\n"
        "v = inputs.normal(963, (1, 1, 90, 64), 'bf16')\n"
        "got = G.prefill(q, k, v, True, 0.125, 'bf16')\n"
        "f = lambda x: inputs.as_f64(x, 'bf16')\n"
        "err = G.max_err(got, oracle.attention(f(q), f(k), f(v), 0.125, True))\n"
        "assert err <= G.TOL['bf16'], err\n"
        "print('ok', err)\n"
    ) % (str(root), str(root / "tests"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]


def test_decode_split_merge_with_reused_workspace():
    """One workspace, first filled with 0xFF bytes, serves five split decodes
    (the default plan: 19 splits) on different inputs: every output matches the oracle and a
    fresh-workspace call bit for bit (nothing is carried over between
    calls)."""
    import torch
    B, H_q, H_kv, T, D = 4, 32, 8, 3000, 128
    assert abi.attn_fwd_decode_default_splits(B, H_q, H_kv, T, D) == 19
    nbytes = abi.attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T, D, abi.ATTN_BF16, 0)
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
    scale = float(np.float32(1.0 / math.sqrt(D)))
    for i in range(5):
        q = gen(700 + 3 * i, (B, H_q, 1, D), "bf16")
        k = gen(701 + 3 * i, (B, H_kv, T, D), "bf16")
        v = gen(702 + 3 * i, (B, H_kv, T, D), "bf16")
        qd, kd, vd = (G.to_device(x, "bf16") for x in (q, k, v))
        o = torch.empty_like(qd)
        G.note(f"decode with a reused workspace, call {i}")
        abi.attn_fwd_decode(qd, kd, vd, o, B, H_q, H_kv, 1, T, D, False, scale, abi.ATTN_BF16, 0, ws, nbytes,
                            torch.cuda.current_stream())
        torch.cuda.synchronize()
        got = G.to_f64(o, "bf16")
        fresh = G.decode(q, k, v, scale, "bf16")
        assert np.array_equal(got, fresh)
        want = oracle.attention(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), scale, False)
        assert G.max_err(got, want) <= G.TOL["bf16"]


@pytest.mark.parametrize("H_q,H_kv,splits", [(8, 2, 16), (4, 4, 2), (3, 3, 5), (16, 4, 7), (12, 3, 16),
                                             (5, 5, 17), (40, 8, 9)])
def test_decode_split_counts_match_oracle(H_q, H_kv, splits):
    """Split decodes over a range of split counts and group sizes, D = 64 and
    128."""
    for D in (64, 128):
        B, T = 3, 1111
        q = gen(810 + D, (B, H_q, 1, D), "bf16")
        k = gen(811 + D, (B, H_kv, T, D), "bf16")
        v = gen(812 + D, (B, H_kv, T, D), "bf16")
        scale = float(np.float32(1.0 / math.sqrt(D)))
        got = G.decode(q, k, v, scale, "bf16", splits)
        want = oracle.attention(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), scale, False)
        assert G.max_err(got, want) <= G.TOL["bf16"], (H_q, H_kv, splits, D)
