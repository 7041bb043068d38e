"""Seeded synthetic inputs (no attention arithmetic lives here).

Thin ctypes front end of ``csrc/gen/normal_gen.c``: SplitMix64 in counter
mode, Box-Muller in double, then round-to-nearest-even to float32 and, for
bfloat16 tensors, on to bfloat16.  Values are i.i.d. N(0,1), the distribution
the pages assume when they derive the 1/sqrt(d_k) scale (AIInfraGuide
"Self-Attention" page, section 6).

bfloat16 tensors are returned as their uint16 bit patterns, because numpy has
no bfloat16 type; :func:`bf16_bits_to_f32` widens them exactly.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

_LIB_PATH = Path(__file__).resolve().parent / "_lib" / "libattn_gen.so"
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise RuntimeError(
                f"{_LIB_PATH} is missing: run __graft_entry__.build() (or "
                "python -m transformer_scaled_dot_flash_amd.build) first")
        lib = ctypes.CDLL(str(_LIB_PATH))
        u64 = ctypes.c_uint64
        for name in ("attn_gen_normal_f64", "attn_gen_normal_f32", "attn_gen_normal_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [u64, u64, u64, ctypes.c_void_p, ctypes.c_int]
            fn.restype = ctypes.c_int
        lib.attn_gen_splitmix64.argtypes = [u64, u64]
        lib.attn_gen_splitmix64.restype = u64
        _lib = lib
    return _lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def splitmix64(seed: int, index: int) -> int:
    """Output ``index`` (0-based) of the SplitMix64 stream ``seed``."""
    return int(_load().attn_gen_splitmix64(seed, index))


def normal(seed: int, shape, dtype: str = "f32", first: int = 0) -> np.ndarray:
    """i.i.d. N(0,1) tensor of ``shape``; dtype 'f64', 'f32' or 'bf16' (bits)."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    lib = _load()
    if dtype == "f64":
        out = np.empty(shape, np.float64)
        fn = lib.attn_gen_normal_f64
    elif dtype == "f32":
        out = np.empty(shape, np.float32)
        fn = lib.attn_gen_normal_f32
    elif dtype == "bf16":
        out = np.empty(shape, np.uint16)
        fn = lib.attn_gen_normal_bf16
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    if n:
        rc = fn(seed, first, n, out.ctypes.data, _threads())
        if rc != 0:
            raise RuntimeError("input generator failed")
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 round-to-nearest-even, as bit patterns (finite input)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Generator output as float64 values (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)
