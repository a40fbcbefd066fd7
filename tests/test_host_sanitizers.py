"""CPU: the host side of every C-ABI entry point under AddressSanitizer and
UndefinedBehaviorSanitizer.

Every library source is compiled as it is for the GPU build, with the sanitizers on the
host half only (``-Xarch_host``: the gfx950 code objects are built normally).  Two checks
use those objects:

* ``host_sanitize/validation_driver.cpp``, linked with them, makes calls that fail
  validation or only size a workspace: null, shape, stride, dtype, alignment, workspace
  and feasibility errors of each entry point, the static-scratch limit of the decode,
  and the status and timing-mark helpers;
* ``tests/test_host.py`` runs in a child process against a shared library linked from
  them (``KVSLIM_LIBRARY``), with the shared sanitizer runtime preloaded into Python.

None of these calls launches a kernel, so no GPU is needed.  Any sanitizer report or
failed check fails the test.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_kv_kvslimmer_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "host_sanitize", "validation_driver.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]

pytestmark = pytest.mark.skipif(not (os.path.exists(B.HIPCC) and os.path.exists(CLANG) and ASAN_RT),
                                reason="ROCm toolchain with sanitizer runtimes not installed")


def _env():
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations; leaks are not what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _clean(r):
    report = r.stdout + r.stderr
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert r.returncode == 0, report[-4000:]


@pytest.fixture(scope="module")
def objects(tmp_path_factory):
    out = tmp_path_factory.mktemp("kvslim_san")
    flags = ["-O1", "-g", *[f for f in B.FLAGS if f != "-O3"], *SAN]

    def compile_one(src):
        obj = str(out / (src.replace(".", "_") + ".o"))
        cmd = [B.HIPCC, *flags, "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"hipcc failed for {src}:\n{r.stderr[-4000:]}"
        return obj

    jobs = min(len(B.SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    return out, objs


def test_entry_point_validation_is_clean_under_asan_and_ubsan(objects):
    out, objs = objects
    exe = str(out / "validation_driver")
    link = [CLANG, "-g", "-fsanitize=address,undefined", f"-I{os.path.join(B.ROOT, 'include')}",
            "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", DRIVER, *objs,
            f"-L{ROCM_LIB}", f"-Wl,-rpath,{ROCM_LIB}", "-lamdhip64", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stderr[-4000:]}"
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=120)
    _clean(r)
    assert "0 failed checks" in r.stdout


def test_host_tests_pass_on_the_sanitized_library(objects):
    out, objs = objects
    lib = str(out / "libkvslim_san.so")
    link = [CLANG, "-shared", "-fPIC", "-shared-libsan", "-fsanitize=address,undefined", "-o", lib, *objs,
            f"-L{ROCM_LIB}", f"-Wl,-rpath,{ROCM_LIB}", "-lamdhip64"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stderr[-4000:]}"
    env = _env()
    env["KVSLIM_LIBRARY"] = lib
    env["LD_PRELOAD"] = ASAN_RT[-1]
    # the child really maps the sanitized build
    probe = ("from long_context_kv_kvslimmer_amd import kvslim\n"
             f"assert any({lib!r} in l for l in open('/proc/self/maps')), 'sanitized library not loaded'\n")
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True, env=env, cwd=B.ROOT,
                       timeout=300)
    _clean(r)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_host.py"), "-x", "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       capture_output=True, text=True, env=env, cwd=B.ROOT, timeout=600)
    _clean(r)
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
