"""Host-side validation and the seeded generator under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

The C ABI and ``normal_gen.c`` are rebuilt with the host code instrumented
(``build.build_sanitized``; device code as usual).  A child process with the
sanitizer runtime preloaded runs every rejection and empty-problem case of
``test_abi_cpu.py`` against that build and hashes the generator's output;
any sanitizer report aborts the child.  The digests must equal the plain
build's, so the instrumented generator computes the same values.
"""
import os
import subprocess
import sys
from pathlib import Path

import pytest

from transformer_scaled_dot_flash_amd import build

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(Path(__file__).resolve().parent))
import sanitized_abi_run as runner  # noqa: E402

LIBS = ("libattn.so", "libattn_gen.so")


@pytest.fixture(scope="module")
def sandir():
    if build.asan_runtime() is None:
        pytest.skip("clang AddressSanitizer runtime not installed")
    if not all((build.SANDIR / n).exists() for n in LIBS):
        build.build_sanitized()
    return build.SANDIR


def test_sanitized_library_is_instrumented(sandir):
    nm = subprocess.run(["nm", "-D", "--undefined-only", str(sandir / "libattn.so")],
                        capture_output=True, text=True, check=True).stdout
    assert "__asan_report_" in nm, "host code of libattn.so not built with AddressSanitizer"
    assert "__ubsan_handle_" in nm, "host code of libattn.so not built with UBSan"
    nm = subprocess.run(["nm", "-D", "--undefined-only", str(sandir / "libattn_gen.so")],
                        capture_output=True, text=True, check=True).stdout
    assert "__asan_report_" in nm and "__ubsan_handle_" in nm


def test_abi_rejections_and_generator_clean_under_sanitizers(sandir):
    env = dict(os.environ)
    pre = str(build.asan_runtime())
    env["LD_PRELOAD"] = pre + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # the HIP runtime and Python keep allocations until exit: leaks are not checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONPATH"] = str(ROOT) + (os.pathsep + env["PYTHONPATH"] if env.get("PYTHONPATH") else "")
    r = subprocess.run([sys.executable, str(Path(runner.__file__)), str(sandir)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert "sanitized run complete" in r.stdout
    got = [ln.split()[1] for ln in r.stdout.splitlines() if ln.startswith("gen ")]
    assert got == runner.gen_digests(), "instrumented generator output differs from the plain build"
