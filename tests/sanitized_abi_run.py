"""Child-process runner of ``test_sanitize_cpu.py`` (not collected by pytest).

Started with the AddressSanitizer runtime preloaded.  It points the package's
two ctypes loaders at the sanitizer builds in ``argv[1]``, checks that the
runtime is live, runs every case of ``test_abi_cpu.py`` (each invalid call
goes through the C ABI's host-side validation and returns a status before any
HIP call), then prints digests of the seeded generator's output for the
parent to compare with the plain build's.
"""
import ctypes
import hashlib
import sys
from pathlib import Path

import transformer_scaled_dot_flash_amd.attn as A
import transformer_scaled_dot_flash_amd.inputs as I

GEN_CASES = [(7, (3, 5, 129), "f64"), (11, (2, 4, 1000), "f32"), (2024, (4, 8, 333, 64), "bf16"),
             (1, (1,), "f32"), (5, (0,), "f32")]


def gen_digests():
    out = []
    for seed, shape, dt in GEN_CASES:
        x = I.normal(seed, shape, dt)
        out.append(hashlib.sha256(x.tobytes()).hexdigest())
    return out


def main():
    d = Path(sys.argv[1])
    A.LIB_PATH = d / "libattn.so"
    I._LIB_PATH = d / "libattn_gen.so"
    proc = ctypes.CDLL(None)
    assert hasattr(proc, "__asan_init"), "AddressSanitizer runtime not loaded"
    import pytest
    here = Path(__file__).resolve().parent
    rc = pytest.main(["-q", "-p", "no:cacheprovider", str(here / "test_abi_cpu.py")])
    if rc != 0:
        return int(rc)
    for h in gen_digests():
        print("gen", h)
    print("sanitized run complete")
    return 0


if __name__ == "__main__":
    sys.exit(main())
