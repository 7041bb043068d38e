"""attn_fwd_decode_noalloc (static device scratch, no workspace argument)
against attn_fwd_decode with a caller-owned workspace: the same kernels and
split plan, so the outputs must agree bit for bit.  Two calls in a row, the
second smaller, so the second call runs over the first call's leftovers in
the shared scratch."""
import math

import numpy as np
import pytest

import gpu_util as G
import oracle
from transformer_scaled_dot_flash_amd import attn as abi
from transformer_scaled_dot_flash_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    abi.load_library()


def _pair(q, k, v, B, H_q, H_kv, T_kv, D, scale, code, splits, stream):
    """(O from attn_fwd_decode with a workspace, O from the no-allocation
    entry point), both on `stream`."""
    torch = G.torch_mod()
    o_ws = torch.full_like(q, float("nan"))
    o_na = torch.full_like(q, float("nan"))
    n = abi.attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T_kv, D, code, splits)
    assert n <= 16 << 20
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    G.note(f"decode (workspace) B={B} H_q={H_q} H_kv={H_kv} T_kv={T_kv} D={D} splits={splits} ws={n}")
    abi.attn_fwd_decode(q, k, v, o_ws, B, H_q, H_kv, 1, T_kv, D, False, scale, code, splits, ws, n,
                        stream)
    G.note(f"decode_noalloc B={B} H_q={H_q} H_kv={H_kv} T_kv={T_kv} D={D} splits={splits}")
    abi.attn_fwd_decode_noalloc(q, k, v, o_na, B, H_q, H_kv, 1, T_kv, D, False, scale, code, splits,
                                stream)
    torch.cuda.synchronize()
    return o_ws, o_na


def test_noalloc_matches_workspace_decode_twice():
    torch = G.torch_mod()
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(4242)
    # 1: long-context decode whose default plan splits the keys (24 splits)
    B, H_q, H_kv, T_kv, D = 4, 32, 8, 32768, 128
    assert abi.attn_fwd_decode_default_splits(B, H_q, H_kv, T_kv, D) > 1
    q = torch.randn(B, H_q, 1, D, device="cuda", generator=g).to(torch.bfloat16)
    k = torch.randn(B, H_kv, T_kv, D, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(B, H_kv, T_kv, D, device="cuda", generator=g).to(torch.bfloat16)
    scale = float(np.float32(1 / math.sqrt(D)))
    o_ws, o_na = _pair(q, k, v, B, H_q, H_kv, T_kv, D, scale, abi.ATTN_BF16, 0, stream)
    assert torch.isfinite(o_ws.float()).all()
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    # 2: a smaller call over the leftovers of the first (D = 64, 5 splits), also
    # checked against the oracle at the bf16 bar
    B, H_q, H_kv, T_kv, D = 2, 16, 4, 3000, 64
    qa = inputs.normal(9101, (B, H_q, 1, D), "bf16")
    ka = inputs.normal(9102, (B, H_kv, T_kv, D), "bf16")
    va = inputs.normal(9103, (B, H_kv, T_kv, D), "bf16")
    qd, kd, vd = (G.to_device(x, "bf16") for x in (qa, ka, va))
    scale = float(np.float32(1 / math.sqrt(D)))
    o_ws, o_na = _pair(qd, kd, vd, B, H_q, H_kv, T_kv, D, scale, abi.ATTN_BF16, 5, stream)
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    want = oracle.attention(inputs.as_f64(qa, "bf16"), inputs.as_f64(ka, "bf16"),
                            inputs.as_f64(va, "bf16"), scale, False)
    assert G.max_err(G.to_f64(o_na, "bf16"), want) <= G.TOL["bf16"]


def test_noalloc_on_a_side_stream_and_single_split():
    torch = G.torch_mod()
    side = torch.cuda.Stream()  # default priority
    g = torch.Generator(device="cuda").manual_seed(77)
    for (B, H_q, H_kv, T_kv, D, splits) in [(1, 8, 2, 5000, 128, 0), (3, 8, 8, 700, 128, 1),
                                            (1, 64, 1, 4097, 128, 7)]:
        q = torch.randn(B, H_q, 1, D, device="cuda", generator=g).to(torch.bfloat16)
        k = torch.randn(B, H_kv, T_kv, D, device="cuda", generator=g).to(torch.bfloat16)
        v = torch.randn(B, H_kv, T_kv, D, device="cuda", generator=g).to(torch.bfloat16)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            o_ws, o_na = _pair(q, k, v, B, H_q, H_kv, T_kv, D, 0.088, abi.ATTN_BF16, splits, side)
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), (B, H_q, H_kv, T_kv, splits)


def test_noalloc_f32_matches():
    torch = G.torch_mod()
    g = torch.Generator(device="cuda").manual_seed(5)
    B, H_q, H_kv, T_kv, D = 2, 8, 2, 333, 64
    q = torch.randn(B, H_q, 1, D, device="cuda", generator=g)
    k = torch.randn(B, H_kv, T_kv, D, device="cuda", generator=g)
    v = torch.randn(B, H_kv, T_kv, D, device="cuda", generator=g)
    o_ws, o_na = _pair(q, k, v, B, H_q, H_kv, T_kv, D, 0.125, abi.ATTN_F32, 0, torch.cuda.current_stream())
    assert torch.equal(o_ws, o_na)
