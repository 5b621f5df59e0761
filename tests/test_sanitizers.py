"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code.

* The oracle (plain C, gcc): oracle/sanitize_check.c drives every exported
  routine on small inputs with exactly sized buffers (ragged segments, a
  width that is not a power of two, empty sequences).
* The library's argument validation and work-space arithmetic (hipcc, the
  sanitizers on the host side only; the device code is built as usual):
  tests/abi_host_check.cpp calls every entry point with arguments its checks
  must refuse before any device work, and every work-space query over sizes
  up to about 2^31 token-heads.  No GPU is touched.

CPU tests; each skips when its compiler is absent.  The library build takes
about a minute and a half (the device code of every source is compiled).
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunkwise_gated_delta_gdn_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on the host pass only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{cmd[0]} failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitize_check")
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    _run([gcc, "-O1", "-g", *san, "-std=c99", "-Wall", "-Wno-unknown-pragmas", "-o", exe,
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), os.path.join(ROOT, "oracle", "sanitize_check.c"), "-lm"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "all routines clean" in r.stdout


def test_library_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *flags, "-x", "hip", "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 4, 8)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_host_check.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", *HOST_SAN, "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "abi_host_check.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_host_check")
    _run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, "-o", exe, drv, *objs])
    # the HIP runtime's own allocations outlive main: leak checking is off
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "all checks passed" in r.stdout
