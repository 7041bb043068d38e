"""The torch front end checks, before anything reaches the GPU, that every
tensor has the shape, dtype and device the C ABI's integer arguments will
describe (the ABI sizes buffers from those integers, so a mismatch would
read or write past a tensor's end).  CPU tensors: a mismatch raises its own
error; a consistent call gets as far as the device check."""
import pytest

torch = pytest.importorskip("torch")
from transformer_scaled_dot_flash_amd import ops_torch as ops  # noqa: E402

bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


GPU = "must be a GPU tensor"


@pytest.mark.parametrize("q,k,v,out,err,match", [
    (t(2, 8, 64, 128), t(2, 2, 64, 128), t(2, 2, 64, 128), None, ValueError, GPU),
    (t(2, 8, 64, 128), t(1, 2, 64, 128), t(1, 2, 64, 128), None, ValueError, "batch"),
    (t(2, 8, 64, 128), t(2, 2, 64, 64), t(2, 2, 64, 64), None, ValueError, "head dim"),
    (t(2, 8, 64, 128), t(2, 3, 64, 128), t(2, 3, 64, 128), None, ValueError, "multiple"),
    (t(2, 8, 64, 128), t(2, 2, 64, 128), t(2, 2, 65, 128), None, ValueError, "differ"),
    (t(2, 8, 64, 128), t(2, 2, 64, 128), t(2, 2, 64, 128, dtype=torch.float32), None, TypeError, "dtype"),
    (t(8, 64, 128), t(2, 2, 64, 128), t(2, 2, 64, 128), None, ValueError, "4-D"),
    (t(2, 8, 64, 128), t(2, 2, 64, 128), t(2, 2, 64, 128), t(2, 8, 63, 128), ValueError, "out has shape"),
    (t(2, 8, 64, 128), t(2, 2, 64, 128), t(2, 2, 64, 128), t(2, 8, 64, 128, dtype=torch.float32),
     TypeError, "out has dtype"),
    (t(2, 8, 64, 128, dtype=torch.float16), t(2, 2, 64, 128, dtype=torch.float16),
     t(2, 2, 64, 128, dtype=torch.float16), None, TypeError, "unsupported dtype"),
])
def test_prefill_and_window_check_shapes_first(q, k, v, out, err, match):
    with pytest.raises(err, match=match):
        ops.prefill(q, k, v, True, 0.1, out=out)
    with pytest.raises(err, match=match):
        ops.prefill_window(q, k, v, 16, 0.1, out=out)


@pytest.mark.parametrize("q,k,out,match", [
    (t(4, 8, 1, 128), t(4, 2, 300, 128), None, GPU),
    (t(4, 8, 2, 128), t(4, 2, 300, 128), None, "one query row"),
    (t(4, 8, 1, 128), t(3, 2, 300, 128), None, "batch"),
    (t(4, 8, 1, 64), t(4, 2, 300, 128), None, "head dim"),
    (t(4, 8, 1, 128), t(4, 2, 300, 128), t(4, 8, 1, 64), "out has shape"),
])
def test_decode_checks_shapes_first(q, k, out, match):
    with pytest.raises(ValueError, match=match):
        ops.decode(q, k, k.clone(), 0.1, out=out)


def paged_args(B=2, H_q=8, H_kv=2, D=128, ps=16, n_pages=40, max_pages=12):
    return dict(q=t(B, H_q, D), k_pages=t(n_pages, H_kv, ps, D), v_pages=t(n_pages, H_kv, ps, D),
                block_table=t(B, max_pages, dtype=torch.int32), seq_lens=t(B, dtype=torch.int32))


@pytest.mark.parametrize("change,err,match", [
    ({}, ValueError, GPU),
    ({"block_table": t(3, 12, dtype=torch.int32)}, ValueError, "block_table"),
    ({"block_table": t(24, dtype=torch.int32)}, ValueError, "block_table"),
    ({"seq_lens": t(3, dtype=torch.int32)}, ValueError, "seq_lens"),
    ({"seq_lens": t(2, dtype=torch.int64)}, TypeError, "int32"),
    ({"q": t(2, 8, 64)}, ValueError, "head dim"),
    ({"q": t(2, 8, 2, 128)}, ValueError, "one query row"),
    ({"v_pages": t(40, 2, 32, 128)}, ValueError, "k_pages and v_pages"),
    ({"out": t(2, 8, 64)}, ValueError, "out has shape"),
])
def test_decode_paged_checks_shapes_first(change, err, match):
    a = paged_args()
    out = change.pop("out", None)
    a.update(change)
    with pytest.raises(err, match=match):
        ops.decode_paged(a["q"], a["k_pages"], a["v_pages"], a["block_table"], a["seq_lens"], 0.1, out=out)


@pytest.mark.parametrize("change,err,match", [
    ({}, ValueError, GPU),
    ({"k": t(300, 2, 64)}, ValueError, "shape|head dim"),
    ({"cu_k": t(5, dtype=torch.int32)}, ValueError, "cu_seqlens"),
    ({"cu_q": t(4, dtype=torch.int64)}, TypeError, "int32"),
    ({"out": t(299, 8, 128)}, ValueError, "out has shape"),
    ({"q": t(300, 8, 128, dtype=torch.float32)}, TypeError, "dtype"),
])
def test_varlen_checks_shapes_first(change, err, match):
    a = dict(q=t(300, 8, 128), k=t(300, 2, 128), v=t(300, 2, 128), cu_q=t(4, dtype=torch.int32),
             cu_k=t(4, dtype=torch.int32))
    out = change.pop("out", None)
    a.update(change)
    if "k" in change:
        a["v"] = a["k"].clone()
    with pytest.raises(err, match=match):
        ops.prefill_varlen(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], 200, 200, True, 0.1, out=out)


@pytest.mark.parametrize("x,w,match", [
    (t(200, 256), t(12 * 64, 256), GPU),
    (t(199, 256), t(12 * 64, 256), "rows"),
    (t(200, 256), t(12 * 64, 192), "w has shape"),
    (t(200, 256), t(11 * 64, 256), "w has shape"),
    (t(200, 256, 1), t(12 * 64, 256), "2-D"),
])
def test_qkv_project_checks_shapes_first(x, w, match):
    # B=2, T=100, H_q=8, H_kv=2, D=64: W has (8 + 2*2) * 64 rows
    with pytest.raises(ValueError, match=match):
        ops.qkv_project(x, w, 2, 100, 8, 2, 64)
