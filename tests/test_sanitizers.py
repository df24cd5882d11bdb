"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

- The oracle's C code, driven over small random inputs and edge cases
  (tests/sanitize/or_driver.c): every entry point, bad tokens and
  temperatures, -inf / +inf / NaN rows, malformed trees, both sibling rules.
- The library's host code: every source compiled with the sanitizers on its
  host side only (the device code is built as usual), linked with a driver
  that calls every C-ABI entry point with invalid arguments and with empty
  batches (tests/sanitize/api_driver.cpp). Those calls return before any HIP
  call, so no GPU is needed; the driver also sizes workspaces at the largest
  shapes.
Any sanitizer report aborts the driver and fails the test."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "rejection_sampling_verify_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "or_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-fopenmp", os.path.join(HERE, "or_driver.c"),
          os.path.join(ROOT, "oracle", "sv_oracle.c"), "-lm", "-o", exe])
    _run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))


def test_library_host_code_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not available")
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

    def compile_one(f):
        obj = str(tmp_path / f.replace(".hip", ".o"))
        _run([HIPCC, *flags, "-c", os.path.join(CSRC, f), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "api_driver")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(HERE, "api_driver.cpp"), *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    _run([exe], env=SAN_ENV)
