"""CPU: the host side of every C-ABI entry point under AddressSanitizer and
UndefinedBehaviorSanitizer.

Every library source is compiled as it is for the GPU build, with the sanitizers on the
host half only (``-Xarch_host``: the gfx950 code objects are built normally), and linked
into ``host_sanitize/validation_driver.cpp``.  The driver makes calls that fail
validation or only size a workspace: null, shape, stride, dtype, alignment, workspace
and feasibility errors of each entry point, the static-scratch limit of the decode, and
the status and timing-mark helpers.  None of these calls launches a kernel, so the test
needs no GPU.  Any sanitizer report or failed check fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_kv_kvslimmer_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host_sanitize", "validation_driver.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _flags():
    # the library's own flags at -O1 -g, with the host half sanitized
    out = [f for f in B.FLAGS if f != "-O3"]
    return ["-O1", "-g", *out, *SAN]


@pytest.mark.skipif(not (os.path.exists(B.HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not installed")
def test_entry_point_validation_is_clean_under_asan_and_ubsan(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (src.replace(".", "_") + ".o"))
        cmd = [B.HIPCC, *_flags(), "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"hipcc failed for {src}:\n{r.stderr[-4000:]}"
        return obj

    jobs = min(len(B.SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    exe = str(tmp_path / "validation_driver")
    link = [CLANG, "-g", "-fsanitize=address,undefined", f"-I{os.path.join(B.ROOT, 'include')}",
            "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", DRIVER, *objs,
            f"-L{ROCM_LIB}", f"-Wl,-rpath,{ROCM_LIB}", "-lamdhip64", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stderr[-4000:]}"

    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations; leaks are not what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    report = r.stdout + r.stderr
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]
    assert "0 failed checks" in r.stdout
    shutil.rmtree(tmp_path, ignore_errors=True)
