"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects every invalid call on the host, before any HIP call
(so no GPU is needed).  No compute call is made here."""
import ctypes
import re
from pathlib import Path

import pytest

import transformer_scaled_dot_flash_amd.attn as A

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "attn.h"

OK, NULL, SHAPE, UNSUP, SCALE, ALIGN, ALIAS, WS, HIP, SCRATCH = range(10)
BF16, F32 = A.ATTN_BF16, A.ATTN_F32

# Fake, well-separated, 16-byte aligned device addresses: never dereferenced,
# because every call below fails validation (or is empty) before any HIP call.
QP, KP, VP, OP, WP = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def header_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(str(A.LIB_PATH))
    declared = header_functions()
    assert declared, "no functions found in the header"
    assert set(declared) == set(A.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in attn.h but not exported"


def test_version_and_strings():
    assert A.attn_abi_version() == 2
    for st in range(10):
        assert A.attn_status_string(st) and A.attn_status_string(st) != "unknown status"
    assert A.attn_status_string(99) == "unknown status"


def prefill(q=QP, k=KP, v=VP, o=OP, B=1, H_q=4, H_kv=4, T_q=128, T_kv=128, D=64, causal=1,
            scale=0.125, dtype=BF16):
    return A.attn_fwd_prefill(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, causal, scale, dtype,
                              None, check=False)


def decode(q=QP, k=KP, v=VP, o=OP, B=2, H_q=8, H_kv=2, T_q=1, T_kv=300, D=128, scale=0.1,
           dtype=BF16, splits=0, ws=WP, ws_bytes=1 << 30):
    return A.attn_fwd_decode(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, 0, scale, dtype, splits,
                             ws, ws_bytes, None, check=False)


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), SHAPE), (dict(H_q=0), SHAPE), (dict(H_kv=0), SHAPE), (dict(T_q=-5), SHAPE),
    (dict(T_kv=0), SHAPE), (dict(H_q=6, H_kv=4), SHAPE), (dict(causal=1, T_q=129, T_kv=128), SHAPE),
    (dict(D=96), UNSUP), (dict(D=256), UNSUP), (dict(dtype=7), UNSUP),
    (dict(scale=float("nan")), SCALE), (dict(scale=float("inf")), SCALE),
    (dict(q=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL), (dict(o=0), NULL),
    (dict(q=QP + 8), ALIGN), (dict(o=OP + 2), ALIGN),
    (dict(o=QP), ALIAS), (dict(o=KP + 64), ALIAS), (dict(o=VP - 1024), ALIAS),
    (dict(B=70000, H_q=70000, H_kv=70000), SHAPE),
    (dict(T_kv=1 << 24, D=128, causal=0), SHAPE),
])
def test_prefill_rejects(kw, want):
    assert prefill(**kw) == want


def test_prefill_checks_params_before_pointers():
    # an invalid shape wins over a null pointer
    assert prefill(q=0, H_q=6, H_kv=4) == SHAPE
    assert prefill(q=0, D=80) == UNSUP


@pytest.mark.parametrize("kw", [dict(B=0), dict(T_q=0, causal=1), dict(T_q=0, causal=0)])
def test_prefill_empty_problem_is_ok_without_pointers(kw):
    assert prefill(q=0, k=0, v=0, o=0, **kw) == OK


def test_prefill_accepts_any_finite_scale():
    # negative and zero scales pass validation; check via an empty problem
    for s in (0.0, -3.5, 1e30):
        assert prefill(B=0, scale=s) == OK


@pytest.mark.parametrize("kw,want", [
    (dict(T_q=2), UNSUP), (dict(T_q=0), UNSUP), (dict(splits=-1), UNSUP), (dict(splits=1025), UNSUP),
    (dict(D=32), UNSUP), (dict(H_q=8, H_kv=3), SHAPE), (dict(T_kv=0), SHAPE),
    (dict(scale=float("-inf")), SCALE), (dict(q=0), NULL), (dict(o=QP), ALIAS),
    (dict(ws=0), WS), (dict(ws_bytes=16), WS), (dict(ws=WP + 4), ALIGN),
    (dict(ws=OP), ALIAS), (dict(ws=KP), ALIAS),
])
def test_decode_rejects(kw, want):
    assert decode(**kw) == want


def test_decode_single_split_needs_no_workspace():
    # With one split requested the split pass writes O and no workspace is
    # used, so a NULL workspace passes validation.  Checked with an empty
    # batch so no kernel is launched.
    assert A.attn_fwd_decode_workspace_bytes(2, 8, 2, 300, 128, BF16, 1) == 0
    assert decode(B=0, ws=0, ws_bytes=0, splits=1) == OK


def test_decode_empty_batch_ok():
    assert decode(B=0, q=0, k=0, v=0, o=0, ws=0, ws_bytes=0) == OK


def ws_expected(B, H_q, H_kv, S, D):
    """(D + 2) fp32 values per (batch, q head, split); 0 for one split."""
    if S <= 1:
        return 0
    return B * H_q * S * (D + 2) * 4


def test_decode_workspace_size():
    B, H_q, H_kv, T_kv, D = 64, 32, 8, 4096, 128
    n = A.attn_fwd_decode_default_splits(B, H_q, H_kv, T_kv, D)
    assert n == 1  # 512 (batch, kv head) groups fill the GPU: no split, no workspace
    assert A.attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T_kv, D, BF16, 0) == 0
    for req, eff in [(1, 0), (8, 8), (64, 64), (128, 128), (4096, 0)]:
        got = A.attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T_kv, D, BF16, req)
        assert got == ws_expected(B, H_q, H_kv, eff, D)  # 0 for one split or an out-of-range request
    # few groups: the keys are split to fill the GPU
    assert A.attn_fwd_decode_default_splits(1, 32, 8, 4096, 128) == 32
    # split count is clamped to the number of 32-key blocks and never leaves a split empty
    assert A.attn_fwd_decode_workspace_bytes(1, 4, 1, 100, 64, BF16, 64) == ws_expected(1, 4, 1, 4, 64)
    assert A.attn_fwd_decode_workspace_bytes(1, 4, 1, 100, 64, BF16, 3) == ws_expected(1, 4, 1, 2, 64)
    assert A.attn_fwd_decode_workspace_bytes(1, 4, 1, 100, 64, F32, 0) == 0
    assert A.attn_fwd_decode_workspace_bytes(1, 4, 3, 100, 64, BF16, 0) == 0
    assert A.attn_fwd_decode_workspace_bytes(1, 64, 1, 4096, 128, BF16, 8) == ws_expected(1, 64, 1, 8, 128)


def default_plan(B, H_q, H_kv, T_kv, D):
    """The default split rule written out: one round of waves (768 at D =
    128, 1024 at D = 64) over the (batch, kv head, 32-head block) groups, at
    least one split and at most one per 4 blocks of 32 keys, then whole
    blocks per split with no empty split."""
    groups = B * H_kv * -(-(H_q // H_kv) // 32)
    blocks = -(-T_kv // 32)
    n = (1024 if D == 64 else 768) // groups
    n = max(1, min(n, max(1, blocks // 4), 1024))
    per = -(-blocks // n)
    return -(-T_kv // (per * 32))


@pytest.mark.parametrize("shape", [(4, 32, 8, 32768, 128), (64, 32, 8, 4096, 128), (64, 32, 8, 4096, 64),
                                   (2, 16, 4, 20000, 64), (16, 32, 8, 8192, 128), (1, 32, 8, 131072, 128),
                                   (32, 32, 8, 4096, 128), (3, 64, 1, 4097, 128), (4, 32, 8, 3000, 128),
                                   (1, 1, 1, 1, 64), (1, 8, 1, 200, 128), (1000, 8, 8, 9000, 64)])
def test_decode_default_split_rule(shape):
    assert A.attn_fwd_decode_default_splits(*shape) == default_plan(*shape)


def test_decode_workspace_too_small_by_one_byte():
    need = A.attn_fwd_decode_workspace_bytes(2, 8, 2, 300, 128, BF16, 0)
    assert decode(ws_bytes=need - 1) == WS


def decode_noalloc(q=QP, k=KP, v=VP, o=OP, B=2, H_q=8, H_kv=2, T_q=1, T_kv=300, D=128, scale=0.1,
                   dtype=BF16, splits=0):
    return A.attn_fwd_decode_noalloc(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, 0, scale, dtype, splits,
                                     None, check=False)


SCRATCH_BYTES = 16 << 20


@pytest.mark.parametrize("kw,want", [
    (dict(T_q=2), UNSUP), (dict(splits=-1), UNSUP), (dict(splits=1025), UNSUP), (dict(D=32), UNSUP),
    (dict(H_q=8, H_kv=3), SHAPE), (dict(T_kv=0), SHAPE), (dict(scale=float("nan")), SCALE),
    (dict(q=0), NULL), (dict(o=0), NULL), (dict(v=VP + 8), ALIGN), (dict(o=KP + 32), ALIAS),
    # 64 * 32 * 64 splits * 130 fp32 = 68 MB of partials: more than the static scratch
    (dict(B=64, H_q=32, H_kv=8, T_kv=4096, splits=64, q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40),
     SCRATCH),
])
def test_decode_noalloc_rejects(kw, want):
    assert decode_noalloc(**kw) == want


def test_decode_noalloc_scratch_limit_is_exact():
    # the largest plan that fits is accepted by validation (checked on an
    # empty batch: nothing launched); one split more needs too much
    B, H_q, H_kv, T_kv, D = 4, 32, 8, 1 << 20, 128
    sizes = {S: A.attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T_kv, D, BF16, S) for S in range(2, 1025)}
    fits = max(S for S, n in sizes.items() if n <= SCRATCH_BYTES)
    assert sizes[fits] <= SCRATCH_BYTES < sizes[fits + 1]
    far = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40)  # 1 GiB K and V: well apart
    assert decode_noalloc(B=B, H_q=H_q, H_kv=H_kv, T_kv=T_kv, splits=fits + 1, **far) == SCRATCH
    assert decode_noalloc(B=0, H_q=H_q, H_kv=H_kv, T_kv=T_kv, splits=fits, q=0, k=0, v=0, o=0) == OK


def test_decode_noalloc_default_plans_fit_the_scratch():
    # the default split plan of every shape with up to 64 q heads per kv head
    # needs at most ~8.5 MiB of partials, within the static scratch
    worst = 0
    for B in (1, 2, 3, 4, 8, 16, 64):
        for H_kv in (1, 2, 8):
            for G in (1, 4, 8, 32, 64):
                for T in (64, 4096, 32768, 1 << 20):
                    worst = max(worst, A.attn_fwd_decode_workspace_bytes(B, G * H_kv, H_kv, T, 128,
                                                                         BF16, 0))
    assert 0 < worst <= SCRATCH_BYTES


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        A.load_library(tmp_path / "libattn.so")


# --- paged decode -------------------------------------------------------------------
TP, SP = 0x60000000, 0x70000000  # fake block table / seq_lens addresses


def paged(q=QP, k=KP, v=VP, o=OP, table=TP, lens=SP, B=2, H_q=8, H_kv=2, D=128, ps=16,
          num_pages=64, max_pages=8, scale=0.1, dtype=BF16, splits=0, ws=WP, ws_bytes=1 << 30):
    return A.attn_fwd_decode_paged(q, k, v, o, table, lens, B, H_q, H_kv, D, ps, num_pages,
                                   max_pages, scale, dtype, splits, ws, ws_bytes, None, check=False)


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), SHAPE), (dict(H_q=0), SHAPE), (dict(H_q=6, H_kv=4), SHAPE),
    (dict(num_pages=0), SHAPE), (dict(max_pages=0), SHAPE),
    (dict(max_pages=1 << 20, ps=4096), SHAPE),
    (dict(ps=8), UNSUP), (dict(ps=24), UNSUP), (dict(ps=1 << 17), UNSUP),
    (dict(dtype=F32), UNSUP), (dict(D=96), UNSUP), (dict(splits=1025), UNSUP),
    (dict(scale=float("nan")), SCALE),
    (dict(q=0), NULL), (dict(table=0), NULL), (dict(lens=0), NULL), (dict(v=0), NULL),
    (dict(q=QP + 8), ALIGN), (dict(table=TP + 2), ALIGN), (dict(lens=SP + 1), ALIGN),
    (dict(o=TP), ALIAS), (dict(o=KP + 16), ALIAS), (dict(ws=SP, max_pages=64), ALIAS),
    (dict(ws=0, max_pages=64), WS), (dict(ws_bytes=15, max_pages=64), WS),
])
def test_paged_rejects(kw, want):
    assert paged(**kw) == want


def test_paged_table_and_lens_only_need_4_byte_alignment():
    # 4-byte aligned table / lengths pass validation (checked with B = 0: no launch)
    assert paged(B=0, table=TP + 4, lens=SP + 4) == OK
    assert paged(B=0, q=0, k=0, v=0, o=0, table=0, lens=0) == OK


def test_paged_workspace_size():
    # one split (enough groups) -> no workspace; few groups -> split over max_pages * ps keys
    assert A.attn_fwd_decode_paged_workspace_bytes(64, 32, 8, 128, 16, 256, 0) == 0
    n = A.attn_fwd_decode_paged_workspace_bytes(1, 32, 8, 128, 16, 256, 0)
    assert n == ws_expected(1, 32, 8, A.attn_fwd_decode_default_splits(1, 32, 8, 4096, 128), 128)
    assert A.attn_fwd_decode_paged_workspace_bytes(2, 8, 2, 128, 16, 8, 4) == \
        A.attn_fwd_decode_workspace_bytes(2, 8, 2, 128, 128, BF16, 4)
    assert A.attn_fwd_decode_paged_workspace_bytes(2, 8, 2, 128, 12, 8, 4) == 0  # bad page size
    need = A.attn_fwd_decode_paged_workspace_bytes(2, 8, 2, 128, 16, 64, 0)
    assert need > 0 and paged(max_pages=64, ws_bytes=need - 1) == WS


# --- sliding window and packed prefill ------------------------------------------------
def window(q=QP, k=KP, v=VP, o=OP, B=1, H_q=4, H_kv=2, T_q=128, T_kv=128, D=64, W=16,
           scale=0.1, dtype=BF16):
    return A.attn_fwd_prefill_window(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, W, scale, dtype, None,
                                     check=False)


@pytest.mark.parametrize("kw,want", [
    (dict(W=0), UNSUP), (dict(W=-3), UNSUP), (dict(dtype=F32), UNSUP), (dict(D=32), UNSUP),
    (dict(T_q=129), SHAPE), (dict(H_q=3), SHAPE), (dict(scale=float("inf")), SCALE),
    (dict(q=0), NULL), (dict(o=VP), ALIAS), (dict(k=KP + 4), ALIGN),
])
def test_window_rejects(kw, want):
    assert window(**kw) == want


def test_window_empty_ok():
    assert window(B=0, q=0, k=0, v=0, o=0) == OK
    assert window(T_q=0, q=0, k=0, v=0, o=0) == OK


CQ, CK = 0x60000000, 0x70000000  # fake cu_seqlens addresses


def varlen(q=QP, k=KP, v=VP, o=OP, cq=CQ, ck=CK, B=3, H_q=8, H_kv=2, D=128, total_q=300,
           total_k=300, mq=200, mk=200, causal=1, W=0, scale=0.1, dtype=BF16):
    return A.attn_fwd_prefill_varlen(q, k, v, o, cq, ck, B, H_q, H_kv, D, total_q, total_k, mq, mk,
                                     causal, W, scale, dtype, None, check=False)


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), SHAPE), (dict(H_kv=3), SHAPE), (dict(total_q=-1), SHAPE), (dict(mq=-2), SHAPE),
    (dict(mq=1 << 20), SHAPE), (dict(mk=1 << 23), SHAPE),
    (dict(dtype=F32), UNSUP), (dict(D=80), UNSUP), (dict(W=-1), UNSUP), (dict(W=8, causal=0), UNSUP),
    (dict(scale=float("nan")), SCALE),
    (dict(q=0), NULL), (dict(cq=0), NULL), (dict(ck=0), NULL),
    (dict(v=VP + 8), ALIGN), (dict(cq=CQ + 2), ALIGN),
    (dict(o=QP), ALIAS), (dict(o=CK - 64), ALIAS),
])
def test_varlen_rejects(kw, want):
    assert varlen(**kw) == want


def test_varlen_empty_ok():
    assert varlen(B=0, q=0, k=0, v=0, o=0, cq=0, ck=0) == OK
    assert varlen(mq=0, q=0, k=0, v=0, o=0, cq=0, ck=0) == OK
    assert varlen(total_q=0, q=0, k=0, v=0, o=0, cq=0, ck=0) == OK
    assert varlen(W=64, causal=1, cq=CQ + 4, ck=CK + 8, B=0) == OK


# --- fused QKV projection ------------------------------------------------------------
XP, WQ, QO, KO, VO = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def qkv(x=XP, w=WQ, q=QO, k=KO, v=VO, B=1, T=128, dm=256, H_q=8, H_kv=2, D=128, dtype=BF16):
    return A.attn_qkv_project(x, w, q, k, v, B, T, dm, H_q, H_kv, D, dtype, None, check=False)


@pytest.mark.parametrize("kw,want", [
    (dict(B=-1), SHAPE), (dict(T=-1), SHAPE), (dict(dm=0), SHAPE), (dict(H_kv=3), SHAPE),
    (dict(T=1 << 20, dm=4096), SHAPE),
    (dict(dm=96), UNSUP), (dict(D=96), UNSUP), (dict(dtype=F32), UNSUP),
    (dict(x=0), NULL), (dict(v=0), NULL), (dict(w=WQ + 4), ALIGN),
    (dict(q=XP), ALIAS), (dict(k=QO + 64), ALIAS), (dict(v=WQ + 256), ALIAS),
])
def test_qkv_rejects(kw, want):
    assert qkv(**kw) == want


def test_qkv_empty_ok():
    assert qkv(B=0, x=0, w=0, q=0, k=0, v=0) == OK
    assert qkv(T=0, x=0, w=0, q=0, k=0, v=0) == OK


# --- measurement probe library ------------------------------------------------------
def test_probe_library_exports_its_header():
    from transformer_scaled_dot_flash_amd import probe
    text = re.sub(r"/\*.*?\*/", "", (ROOT / "include" / "attn_probe.h").read_text(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(attn_probe_[a-z0-9_]+)\s*\(", text)))
    assert set(declared) == set(probe.EXPORTED)
    lib = ctypes.CDLL(str(probe.LIB_PATH))
    for name in declared:
        assert hasattr(lib, name)


def test_probe_rejects_bad_arguments_before_launching():
    from transformer_scaled_dot_flash_amd import probe
    lib = probe.load_library()
    inval = 1  # hipErrorInvalidValue
    assert lib.attn_probe_mfma(0, 10, 0x1000, 0x2000, None) == inval
    assert lib.attn_probe_mfma(4, 10, None, 0x2000, None) == inval
    assert lib.attn_probe_mfma_random(0, 10, 0x1000, 0x2000, None) == inval
    assert lib.attn_probe_mfma_random(4, 0, 0x1000, 0x2000, None) == inval
    assert lib.attn_probe_mfma_random(4, 10, 0x1000, None, None) == inval
    assert lib.attn_probe_stream_read(0x1000, 1 << 20, 0x2000, 3, None) == inval   # not a 64 KiB multiple per WG
    assert lib.attn_probe_stream_read(0x1000, 0, 0x2000, 4, None) == inval
    assert lib.attn_probe_stream_read(None, 1 << 26, 0x2000, 4, None) == inval
    assert lib.attn_probe_clock(None, 100, None) == inval
    assert lib.attn_probe_clock(0x1000, 0, None) == inval
