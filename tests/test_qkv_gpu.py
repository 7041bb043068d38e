"""GPU parity of the fused QKV projection (attn_qkv_project) against the
float64 oracle, and of projection + prefill end to end.

Bar (derived from the arithmetic: fp32 accumulation, then one bf16 rounding
of each output): |Y_gpu - Y_oracle| <= 1e-3 + 2^-8 |Y_oracle| element by
element (half a bf16 ulp is 2^-9 relative; the margin covers fp32
accumulation and a rounding flip next to a tie).  Guard bands around each
output catch writes outside it; every element must be written."""
import zlib

import numpy as np
import pytest

import gpu_util as G
import oracle
import oracle.qkv_fp64 as QP
from transformer_scaled_dot_flash_amd import attn as abi
from transformer_scaled_dot_flash_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.load_library()


def make(B, T, dm, H_q, H_kv, D):
    s = zlib.crc32(repr(("qkv", B, T, dm, H_q, H_kv, D)).encode())
    N = (H_q + 2 * H_kv) * D
    x = inputs.normal(s + 1, (B * T, dm), "bf16")
    # weights ~ N(0, 1/d_model): outputs ~ N(0, 1)
    w32 = inputs.bf16_bits_to_f32(inputs.normal(s + 2, (N, dm), "bf16")) / np.float32(np.sqrt(dm))
    w = inputs.f32_to_bf16_bits(w32)
    return x, w


def run(x, w, B, T, dm, H_q, H_kv, D):
    torch = G.torch_mod()
    xd, wd = G.to_device(x, "bf16"), G.to_device(w, "bf16")
    bq, q = G.guarded_output((B, H_q, T, D), "bf16")
    bk, k = G.guarded_output((B, H_kv, T, D), "bf16")
    bv, v = G.guarded_output((B, H_kv, T, D), "bf16")
    G.note(f"attn_qkv_project B={B} T={T} d_model={dm} H_q={H_q} H_kv={H_kv} D={D}")
    abi.attn_qkv_project(xd, wd, q, k, v, B, T, dm, H_q, H_kv, D, abi.ATTN_BF16,
                         torch.cuda.current_stream())
    torch.cuda.synchronize()
    for buf, name in ((bq, "q"), (bk, "k"), (bv, "v")):
        G.check_guards(buf, "bf16", f"qkv {name}")
    return q, k, v


def check(got, want, what):
    assert np.all(np.isfinite(got)), f"{what}: unwritten or non-finite output"
    bound = 1e-3 + np.abs(want) * 2.0 ** -8
    err = np.abs(got - want)
    worst = float(np.max(err - bound))
    assert worst <= 0, f"{what}: max excess {worst:.3e} over the bound (max err {float(err.max()):.3e})"


CASES = [
    # B, T, d_model, H_q, H_kv, D
    (1, 128, 64, 4, 2, 64),
    (2, 100, 256, 8, 2, 128),
    (3, 77, 768, 12, 12, 64),
    (1, 1000, 4096, 32, 8, 128),
    (2, 300, 512, 4, 1, 128),
    (1, 70, 192, 3, 1, 64),        # N = 320: ragged feature tile; 3 k tiles (odd)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}T{}dm{}H{}/{}D{}".format(*c))
def test_qkv_matches_oracle(case):
    B, T, dm, H_q, H_kv, D = case
    x, w = make(*case)
    q, k, v = run(x, w, *case)
    wq, wk, wv = QP.qkv_project(inputs.as_f64(x, "bf16"), inputs.as_f64(w, "bf16"), B, T, H_q, H_kv, D)
    for t, ref, name in ((q, wq, "Q"), (k, wk, "K"), (v, wv, "V")):
        check(G.to_f64(t, "bf16"), ref, f"{case} {name}")


def test_qkv_large_sampled_tokens():
    B, T, dm, H_q, H_kv, D = 1, 8192, 4096, 32, 8, 128
    x, w = make(B, T, dm, H_q, H_kv, D)
    q, k, v = run(x, w, B, T, dm, H_q, H_kv, D)
    toks = [0, 1, 255, 256, 4095, 8000, 8191]
    y = QP.project(inputs.as_f64(x[toks], "bf16"), inputs.as_f64(w, "bf16"))
    qn, kn = H_q * D, H_kv * D
    gq, gk, gv = (G.to_f64(t, "bf16") for t in (q, k, v))
    for i, t in enumerate(toks):
        check(gq[0, :, t].reshape(-1), y[i, :qn], f"Q token {t}")
        check(gk[0, :, t].reshape(-1), y[i, qn:qn + kn], f"K token {t}")
        check(gv[0, :, t].reshape(-1), y[i, qn + kn:], f"V token {t}")


def test_projection_then_prefill_end_to_end():
    # oracle: fp64 projection rounded to bf16 (as the kernel rounds), then the
    # attention oracle; GPU: attn_qkv_project feeding attn_fwd_prefill
    torch = G.torch_mod()
    B, T, dm, H_q, H_kv, D = 1, 300, 512, 8, 2, 64
    x, w = make(B, T, dm, H_q, H_kv, D)
    q, k, v = run(x, w, B, T, dm, H_q, H_kv, D)
    o = torch.empty_like(q)
    scale = 0.125
    abi.attn_fwd_prefill(q, k, v, o, B, H_q, H_kv, T, T, D, True, scale, abi.ATTN_BF16,
                         torch.cuda.current_stream())
    torch.cuda.synchronize()
    rq, rk, rv = QP.qkv_project(inputs.as_f64(x, "bf16"), inputs.as_f64(w, "bf16"), B, T, H_q, H_kv, D)
    rnd = lambda a: inputs.bf16_bits_to_f32(inputs.f32_to_bf16_bits(a.astype(np.float32))).astype(np.float64)
    want = oracle.attention(rnd(rq), rnd(rk), rnd(rv), scale, True)
    err = G.max_err(G.to_f64(o, "bf16"), want)
    assert err <= G.TOL["bf16"], err
