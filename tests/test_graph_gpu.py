"""The C ABI under HIP graph capture: prefill (bf16 key-split and 4-wave
shapes, fp32 row kernel), split decode with its combine pass, and paged
decode are recorded into one graph on a side stream, replayed several times
with eager work and synchronisations in between, and every replay's outputs
must equal the eager calls' outputs bit for bit (same kernels, same
launch configuration).  The entry points make no allocation, no memset and
no synchronising call, so they are capturable."""
import math

import numpy as np
import pytest

from transformer_scaled_dot_flash_amd import attn as abi
from transformer_scaled_dot_flash_amd import inputs

import gpu_util as G

pytestmark = pytest.mark.gpu


def _calls(torch, dev):
    """(name, run(stream), output tensor) for each captured call.  Every
    shape argument is bound when its closure is made (the names are reused
    for the next call)."""
    calls = []

    def bf16(seed, shape):
        return G.to_device(inputs.normal(seed, shape, "bf16"), "bf16")

    def f32(seed, shape):
        return G.to_device(inputs.normal(seed, shape, "f32"), "f32")

    # bf16 prefill, key-split shape (B1 H4 T128 D64 causal) and 4-wave shape (B2 H32/8 T1100 D64)
    for name, (B, Hq, Hkv, T, D) in (("prefill_keysplit", (1, 4, 4, 128, 64)),
                                     ("prefill_4wave", (2, 32, 8, 1100, 64))):
        q, k, v = bf16(11, (B, Hq, T, D)), bf16(12, (B, Hkv, T, D)), bf16(13, (B, Hkv, T, D))
        o = torch.empty_like(q)
        sc = float(np.float32(1 / math.sqrt(D)))
        calls.append((name, lambda s, q=q, k=k, v=v, o=o, a=(B, Hq, Hkv, T, T, D, 1, sc):
                      abi.attn_fwd_prefill(q, k, v, o, *a, abi.ATTN_BF16, s), o))
    # fp32 prefill, one wave per row (single head T128 D64)
    q, k, v = f32(21, (1, 1, 128, 64)), f32(22, (1, 1, 128, 64)), f32(23, (1, 1, 128, 64))
    o = torch.empty_like(q)
    calls.append(("prefill_f32", lambda s, q=q, k=k, v=v, o=o:
                  abi.attn_fwd_prefill(q, k, v, o, 1, 1, 1, 128, 128, 64, 0, 0.125, abi.ATTN_F32, s), o))
    # split decode: 8 splits, partials in a workspace, then the combine pass
    B, Hq, Hkv, T, D = 2, 8, 2, 5000, 128
    q, k, v = bf16(31, (B, Hq, 1, D)), bf16(32, (B, Hkv, T, D)), bf16(33, (B, Hkv, T, D))
    o = torch.empty_like(q)
    wsb = abi.attn_fwd_decode_workspace_bytes(B, Hq, Hkv, T, D, abi.ATTN_BF16, 8)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    calls.append(("decode_split8", lambda s, q=q, k=k, v=v, o=o, ws=ws, wsb=wsb, a=(B, Hq, Hkv, 1, T, D, 0, 0.088):
                  abi.attn_fwd_decode(q, k, v, o, *a, abi.ATTN_BF16, 8, ws, wsb, s), o))
    # paged decode: 16-token pages in a shuffled pool
    B, Hq, Hkv, T, D, P = 3, 8, 2, 700, 64, 16
    per = (T + P - 1) // P
    n_pages = B * per + 5
    kp, vp = bf16(41, (n_pages, Hkv, P, D)), bf16(42, (n_pages, Hkv, P, D))
    q = bf16(43, (B, Hq, D))
    o = torch.empty_like(q)
    perm = np.random.default_rng(7).permutation(n_pages)[:B * per].astype(np.int32)
    table = torch.from_numpy(perm.reshape(B, per)).to(dev)
    lens = torch.tensor([T, T - 100, 1], dtype=torch.int32, device=dev)
    wsb = abi.attn_fwd_decode_paged_workspace_bytes(B, Hq, Hkv, D, P, per, 0)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    calls.append(("decode_paged", lambda s, q=q, kp=kp, vp=vp, o=o, table=table, lens=lens, ws=ws, wsb=wsb,
                  a=(B, Hq, Hkv, D, P, n_pages, per, 0.125):
                  abi.attn_fwd_decode_paged(q, kp, vp, o, table, lens, *a, abi.ATTN_BF16, 0, ws, wsb, s), o))
    return calls


def test_graph_replays_equal_eager_calls():
    torch = G.torch_mod()
    dev = torch.device("cuda:0")
    calls = _calls(torch, dev)
    cur = torch.cuda.current_stream(dev)
    G.note("graph: eager reference calls")
    for _, run, o in calls:
        o.fill_(float("nan"))
        run(cur)
    torch.cuda.synchronize()
    eager = [o.clone() for _, _, o in calls]
    for (name, _, _), want in zip(calls, eager):
        assert not torch.isnan(want.float()).any(), f"{name}: eager call left elements unwritten"

    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(cur)
    graph = torch.cuda.CUDAGraph()
    G.note("graph: capture")
    with torch.cuda.graph(graph, stream=side):
        for _, run, _ in calls:
            run(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()

    for rep in range(4):
        for _, _, o in calls:
            o.fill_(float("nan"))  # a fill kernel, outside the graph
        # eager work of the program's own between replays
        x = torch.randn(512, 512, device=dev)
        (x @ x).sum().item()
        G.note(f"graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for (name, _, o), want in zip(calls, eager):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), \
                f"replay {rep}: {name} differs from the eager call"
