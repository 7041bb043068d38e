"""Binding of ``include/attn_probe.h`` (ctypes, marshalling only): the
benchmark's measurement kernels (measured matrix-core and HBM-read ceilings,
shader clock).  Like :mod:`attn`, it raises if the library is missing."""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "_lib" / "libattn_probe.so"
EXPORTED = ("attn_probe_mfma", "attn_probe_mfma_random", "attn_probe_stream_read", "attn_probe_clock")

_lib = None


def load_library(path: Path | str | None = None):
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"probe library not built: {p} is missing (run __graft_entry__.build())")
    try:
        import torch  # noqa: F401  (bind to torch's HIP runtime, see attn.load_library)
    except ImportError:
        pass
    lib = ctypes.CDLL(str(p))
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.attn_probe_mfma.argtypes = [i, i, vp, vp, vp]
    lib.attn_probe_mfma_random.argtypes = [i, i, vp, vp, vp]
    lib.attn_probe_stream_read.argtypes = [vp, sz, vp, i, vp]
    lib.attn_probe_clock.argtypes = [vp, i, vp]
    for f in EXPORTED:
        getattr(lib, f).restype = i
    if path is None:
        _lib = lib
    return lib


def _ptr(x):
    return None if x is None else (x if isinstance(x, int) else int(x.data_ptr()))


def _stream(s):
    return None if s is None else (s if isinstance(s, int) else int(s.cuda_stream))


def _check(rc, where):
    if rc != 0:
        raise RuntimeError(f"{where}: hipError {rc}")


def attn_probe_mfma(n_wg, iters, out, cycles, stream=None):
    _check(load_library().attn_probe_mfma(n_wg, iters, _ptr(out), _ptr(cycles), _stream(stream)), "attn_probe_mfma")


def attn_probe_mfma_random(n_wg, iters, out, cycles, stream=None):
    _check(load_library().attn_probe_mfma_random(n_wg, iters, _ptr(out), _ptr(cycles), _stream(stream)),
           "attn_probe_mfma_random")


def attn_probe_stream_read(src, nbytes, sink, n_wg, stream=None):
    _check(load_library().attn_probe_stream_read(_ptr(src), nbytes, _ptr(sink), n_wg, _stream(stream)),
           "attn_probe_stream_read")


def attn_probe_clock(out, ticks, stream=None):
    _check(load_library().attn_probe_clock(_ptr(out), ticks, _stream(stream)), "attn_probe_clock")
