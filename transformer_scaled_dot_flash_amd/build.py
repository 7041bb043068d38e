"""Compile the native parts in-tree.

* ``_lib/libattn.so``      the HIP kernels for gfx950 and the C ABI
                           (``include/attn.h``), built with hipcc.
* ``_lib/libattn_gen.so``  the seeded input generator (plain C, gcc).
* ``_lib/libattn_probe.so`` measurement kernels of the benchmark (measured
                           ceilings and shader clock, ``include/attn_probe.h``).
* ``_lib/san/``            the C ABI and the generator again, with the host code
                           built under AddressSanitizer and UndefinedBehavior-
                           Sanitizer (CPU tests of the host-side validation).
* ``_lib/c_abi_client``    a plain C client of the C ABI (tests/native), run
                           by a GPU test.

All are rebuilt when :func:`build_all` is called.  Loading code never
builds: it raises if a library is missing.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIBDIR = PKG / "_lib"
INCLUDE = ROOT / "include"

# Kernel sources are compiled assuming no NaN operands (scores of finite
# inputs are never NaN; masked scores are -inf), which lets max/min skip NaN
# canonicalisation.  The ABI layer, which validates inputs, is not.
KERNEL_FLAGS = ["-fno-honor-nans"]
KERNEL_SOURCES = {"prefill_bf16.hip", "prefill_f32.hip", "decode_bf16.hip", "qkv_bf16.hip"}

HIP_SOURCES = [
    CSRC / "attn_api.hip",
    CSRC / "prefill_bf16.hip",
    CSRC / "prefill_f32.hip",
    CSRC / "decode_bf16.hip",
    CSRC / "qkv_bf16.hip",
]
HIP_HEADERS = [CSRC / "kernel_common.h", CSRC / "launch.h", INCLUDE / "attn.h", INCLUDE / "attn_probe.h"]

# gfx950 only.  Packed fp32 VALU ops are switched off for all device code.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd: list[str]) -> None:
    print("[build]", " ".join(str(c) for c in cmd), flush=True)
    subprocess.run([str(c) for c in cmd], check=True)


def build_gen() -> Path:
    LIBDIR.mkdir(exist_ok=True)
    out = LIBDIR / "libattn_gen.so"
    tmp = out.with_suffix(".so.tmp")
    _run(["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-pthread",
          str(CSRC / "gen" / "normal_gen.c"), "-o", str(tmp), "-lm"])
    os.replace(tmp, out)
    return out


def build_hip(jobs: int = 4) -> Path:
    LIBDIR.mkdir(exist_ok=True)
    objdir = LIBDIR / "obj"
    objdir.mkdir(exist_ok=True)
    hipcc = _hipcc()
    objs = []
    procs = []
    for src in HIP_SOURCES:
        obj = objdir / (src.stem + ".o")
        objs.append(obj)
        extra = KERNEL_FLAGS if src.name in KERNEL_SOURCES else []
        cmd = [hipcc, *HIP_FLAGS, *extra, "-I", str(INCLUDE), "-I", str(CSRC), "-c", str(src), "-o", str(obj)]
        print("[build]", " ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
        if len(procs) >= jobs:
            if procs.pop(0).wait() != 0:
                raise subprocess.CalledProcessError(1, "hipcc")
    for p in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(1, "hipcc")
    out = LIBDIR / "libattn.so"
    tmp = out.with_suffix(".so.tmp")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)])
    os.replace(tmp, out)
    return out


def build_probe() -> Path:
    LIBDIR.mkdir(exist_ok=True)
    out = LIBDIR / "libattn_probe.so"
    tmp = out.with_suffix(".so.tmp")
    _run([_hipcc(), *HIP_FLAGS, "-shared", "-I", str(INCLUDE), str(CSRC / "probe" / "ceilings.hip"), "-o", str(tmp)])
    os.replace(tmp, out)
    return out


# Host-side sanitizers only: on hipcc lines every flag goes to the host pass
# (-Xarch_host), device code is built as usual (no GPU sanitizer).
HIPCC_SAN_FLAGS = ["-Xarch_host", "-g",
                   "-Xarch_host", "-fsanitize=address",
                   "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined",
                   "-Xarch_host", "-fno-omit-frame-pointer"]
# the generator is plain C, built by clang for the CPU only
C_SAN_FLAGS = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
SANDIR = LIBDIR / "san"


def asan_runtime() -> Path | None:
    """The clang AddressSanitizer runtime matching hipcc's compiler."""
    found = sorted(Path("/opt/rocm/llvm/lib/clang").glob("*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def build_sanitized(jobs: int = 5) -> Path:
    """``_lib/san/libattn.so`` and ``_lib/san/libattn_gen.so`` with the host code
    instrumented.  They are loaded only by a CPU test, in a child process that
    preloads the sanitizer runtime."""
    SANDIR.mkdir(parents=True, exist_ok=True)
    hipcc = _hipcc()
    host = HIPCC_SAN_FLAGS
    objs, procs = [], []
    for src in HIP_SOURCES:
        obj = SANDIR / (src.stem + ".o")
        objs.append(obj)
        cmd = [hipcc, *HIP_FLAGS, *host, "-I", str(INCLUDE), "-I", str(CSRC), "-c", str(src), "-o", str(obj)]
        print("[build]", " ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd))
        if len(procs) >= jobs:
            if procs.pop(0).wait() != 0:
                raise subprocess.CalledProcessError(1, "hipcc")
    for p in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(1, "hipcc")
    out = SANDIR / "libattn.so"
    tmp = out.with_suffix(".so.tmp")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *host, *map(str, objs), "-o", str(tmp)])
    os.replace(tmp, out)
    clang = Path(hipcc).resolve().parent.parent / "llvm" / "bin" / "clang"
    if not clang.exists():
        clang = Path("/opt/rocm/llvm/bin/clang")
    gen = SANDIR / "libattn_gen.so"
    tmp = gen.with_suffix(".so.tmp")
    _run([clang, "-O2", "-fPIC", "-shared", "-std=c11", "-Wall", "-pthread", *C_SAN_FLAGS,
          str(CSRC / "gen" / "normal_gen.c"), "-o", str(tmp), "-lm"])
    os.replace(tmp, gen)
    return out


def build_c_client() -> Path:
    """``_lib/c_abi_client``: a plain C program that calls the C ABI with
    device memory from the HIP runtime (no torch, no Python); a GPU test runs
    it.  Host code only, built with gcc against ``libattn.so`` beside it."""
    out = LIBDIR / "c_abi_client"
    tmp = out.with_name(out.name + ".tmp")
    rocm = Path(_hipcc()).resolve().parent.parent
    _run(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-I", str(INCLUDE), "-I", str(rocm / "include"),
          "-D__HIP_PLATFORM_AMD__", str(ROOT / "tests" / "native" / "c_abi_client.c"), "-L", str(LIBDIR), "-lattn",
          "-L", str(rocm / "lib"), "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN", f"-Wl,-rpath,{rocm / 'lib'}",
          "-o", str(tmp)])
    os.replace(tmp, out)
    return out


def build_all() -> None:
    build_gen()
    build_hip()
    build_probe()
    build_sanitized()
    build_c_client()


if __name__ == "__main__":
    build_all()
    sys.exit(0)
