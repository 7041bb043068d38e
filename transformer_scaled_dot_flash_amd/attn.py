"""Python binding of the C ABI in ``include/attn.h`` (ctypes, marshalling only).

The functions keep the C names.  Pointer arguments accept an ``int`` device
address or any object with ``data_ptr()`` (a torch tensor); ``stream``
accepts an ``int``/``None`` handle or an object with ``cuda_stream`` (a
``torch.cuda.Stream``).  A non-OK status raises :class:`AttnError`.  Every
step of the computation runs in the HIP library; nothing here computes.

PyTorch is only used by callers for device memory and streams; this module
does not import it.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "_lib" / "libattn.so"

ATTN_F32 = 0
ATTN_BF16 = 1

STATUS_NAMES = {
    0: "ATTN_OK",
    1: "ATTN_ERR_NULL_PTR",
    2: "ATTN_ERR_INVALID_SHAPE",
    3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_INVALID_SCALE",
    5: "ATTN_ERR_ALIGNMENT",
    6: "ATTN_ERR_ALIAS",
    7: "ATTN_ERR_WORKSPACE",
    8: "ATTN_ERR_HIP",
    9: "ATTN_ERR_SCRATCH",
}

EXPORTED = (
    "attn_fwd_prefill",
    "attn_fwd_prefill_window",
    "attn_fwd_prefill_varlen",
    "attn_fwd_decode",
    "attn_fwd_decode_noalloc",
    "attn_fwd_decode_workspace_bytes",
    "attn_fwd_decode_default_splits",
    "attn_fwd_decode_paged",
    "attn_fwd_decode_paged_workspace_bytes",
    "attn_qkv_project",
    "attn_status_string",
    "attn_abi_version",
    "attn_last_hip_error",
)


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str, lib=None):
        self.status = status
        msg = f"{where}: {STATUS_NAMES.get(status, status)}"
        if lib is not None:
            msg += f" ({lib.attn_status_string(status).decode()})"
            if status == 8:
                msg += f", hipError {lib.attn_last_hip_error()}"
        super().__init__(msg)


_lib = None


def load_library(path: Path | str | None = None):
    """Load ``libattn.so`` (built by ``__graft_entry__.build()``).  Raises if it
    is missing: there is no fallback implementation."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"HIP attention library not built: {p} is missing "
                           "(run __graft_entry__.build())")
    # PyTorch ships its own HIP runtime under the same soname.  Loaded first,
    # it is the runtime this library binds to; loaded after this library,
    # torch would bring a second runtime into the process, whose device and
    # stream state this library cannot see (launches then fail with
    # hipErrorNoDevice).  So torch, when installed, is loaded before it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(str(p))
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd_prefill.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_prefill.restype = i
    lib.attn_fwd_prefill_window.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_prefill_window.restype = i
    lib.attn_fwd_prefill_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f,
                                            i, vp]
    lib.attn_fwd_prefill_varlen.restype = i
    lib.attn_fwd_decode.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.attn_fwd_decode.restype = i
    lib.attn_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
    lib.attn_fwd_decode_noalloc.restype = i
    lib.attn_fwd_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.attn_fwd_decode_workspace_bytes.restype = sz
    lib.attn_fwd_decode_default_splits.argtypes = [i, i, i, i, i]
    lib.attn_fwd_decode_default_splits.restype = i
    lib.attn_fwd_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp,
                                          sz, vp]
    lib.attn_fwd_decode_paged.restype = i
    lib.attn_fwd_decode_paged_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.attn_fwd_decode_paged_workspace_bytes.restype = sz
    lib.attn_qkv_project.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.attn_qkv_project.restype = i
    lib.attn_status_string.argtypes = [i]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = i
    lib.attn_last_hip_error.argtypes = []
    lib.attn_last_hip_error.restype = i
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise AttnError(status, where, _lib)


def attn_fwd_prefill(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, causal, scale, dtype, stream=None,
                     check=True) -> int:
    lib = load_library()
    st = lib.attn_fwd_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H_q, H_kv, T_q, T_kv, D,
                              1 if causal else 0, float(scale), dtype, _stream(stream))
    if check:
        _check(st, "attn_fwd_prefill")
    return st


def attn_fwd_prefill_window(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, window, scale, dtype,
                            stream=None, check=True) -> int:
    lib = load_library()
    st = lib.attn_fwd_prefill_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H_q, H_kv, T_q, T_kv, D,
                                     window, float(scale), dtype, _stream(stream))
    if check:
        _check(st, "attn_fwd_prefill_window")
    return st


def attn_fwd_prefill_varlen(q, k, v, o, cu_seqlens_q, cu_seqlens_k, B, H_q, H_kv, D, total_q,
                            total_k, max_seqlen_q, max_seqlen_k, causal, window, scale, dtype,
                            stream=None, check=True) -> int:
    lib = load_library()
    st = lib.attn_fwd_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(cu_seqlens_q),
                                     _ptr(cu_seqlens_k), B, H_q, H_kv, D, total_q, total_k,
                                     max_seqlen_q, max_seqlen_k, 1 if causal else 0, window,
                                     float(scale), dtype, _stream(stream))
    if check:
        _check(st, "attn_fwd_prefill_varlen")
    return st


def attn_fwd_decode(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, causal, scale, dtype, num_splits,
                    workspace, workspace_bytes, stream=None, check=True) -> int:
    lib = load_library()
    st = lib.attn_fwd_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H_q, H_kv, T_q, T_kv, D,
                             1 if causal else 0, float(scale), dtype, num_splits, _ptr(workspace),
                             workspace_bytes, _stream(stream))
    if check:
        _check(st, "attn_fwd_decode")
    return st


def attn_fwd_decode_noalloc(q, k, v, o, B, H_q, H_kv, T_q, T_kv, D, causal, scale, dtype,
                            num_splits, stream=None, check=True) -> int:
    lib = load_library()
    st = lib.attn_fwd_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H_q, H_kv, T_q, T_kv, D,
                                     1 if causal else 0, float(scale), dtype, num_splits,
                                     _stream(stream))
    if check:
        _check(st, "attn_fwd_decode_noalloc")
    return st


def attn_fwd_decode_paged(q, k_pages, v_pages, o, block_table, seq_lens, B, H_q, H_kv, D,
                          page_size, num_pages, max_pages, scale, dtype, num_splits, workspace,
                          workspace_bytes, stream=None, check=True) -> int:
    lib = load_library()
    st = lib.attn_fwd_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o),
                                   _ptr(block_table), _ptr(seq_lens), B, H_q, H_kv, D, page_size,
                                   num_pages, max_pages, float(scale), dtype, num_splits,
                                   _ptr(workspace), workspace_bytes, _stream(stream))
    if check:
        _check(st, "attn_fwd_decode_paged")
    return st


def attn_fwd_decode_paged_workspace_bytes(B, H_q, H_kv, D, page_size, max_pages, num_splits=0) -> int:
    return int(load_library().attn_fwd_decode_paged_workspace_bytes(B, H_q, H_kv, D, page_size,
                                                                     max_pages, num_splits))


def attn_qkv_project(x, w, q, k, v, B, T, d_model, H_q, H_kv, D, dtype, stream=None,
                     check=True) -> int:
    lib = load_library()
    st = lib.attn_qkv_project(_ptr(x), _ptr(w), _ptr(q), _ptr(k), _ptr(v), B, T, d_model, H_q, H_kv,
                              D, dtype, _stream(stream))
    if check:
        _check(st, "attn_qkv_project")
    return st


def attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T_kv, D, dtype, num_splits=0) -> int:
    return int(load_library().attn_fwd_decode_workspace_bytes(B, H_q, H_kv, T_kv, D, dtype, num_splits))


def attn_fwd_decode_default_splits(B, H_q, H_kv, T_kv, D) -> int:
    return int(load_library().attn_fwd_decode_default_splits(B, H_q, H_kv, T_kv, D))


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(status).decode()


def attn_abi_version() -> int:
    return int(load_library().attn_abi_version())


def attn_last_hip_error() -> int:
    return int(load_library().attn_last_hip_error())
