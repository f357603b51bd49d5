"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds of the same sources, instrumented on the host side only:
  * the float64 oracle (gcc), driven by its own pin tests;
  * the library's host code -- argument checks, work planning, workspace
    sizing, the admission accounting and the pool telemetry -- driven by the
    C-ABI tests, which never launch a kernel.
Each runs in a child process with the sanitizer runtime preloaded (Python
itself is not instrumented) and stops at the first report.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_tests(env_extra, tests, tmp_path):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    log = tmp_path / "run.log"
    with open(log, "w") as f:
        rc = subprocess.call([sys.executable, "-m", "pytest", *tests, "-q", "-x", "-s", "-p", "no:cacheprovider",
                              "-m", "not gpu"], cwd=ROOT, env=env, stdout=f, stderr=subprocess.STDOUT)
    text = log.read_text()
    assert rc == 0 and "runtime error" not in text and "ERROR: AddressSanitizer" not in text, text[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call([gcc, "-O1", "-g", "-fPIC", "-shared", "-pthread", "-std=c11", "-Wall",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                           "-o", str(lib), os.path.join(ROOT, "oracle", "pa_oracle.c"), "-lm"])
    runtimes = [subprocess.check_output([gcc, f"-print-file-name={n}"], text=True).strip()
                for n in ("libasan.so", "libubsan.so")]
    _run_tests({"LD_PRELOAD": ":".join(runtimes), "PA_ORACLE_LIB": str(lib)},
               ["tests/test_oracle.py", "tests/test_oracle_pool.py", "tests/test_oracle_norm.py"], tmp_path)


def test_library_host_code_under_asan_ubsan(tmp_path):
    asan = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(HIPCC) or not asan:
        pytest.skip("hipcc or its sanitizer runtime not available")
    lib = tmp_path / "libpagedattn_san.so"
    srcs = [os.path.join(ROOT, "paged_kv_decode_slot_amd", "csrc", f)
            for f in ("pagedattn.hip", "blockpool.hip", "rmsnorm.hip", "probe.hip")]
    # Device code is built plainly (and unoptimised, to build fast: no kernel runs here);
    # the sanitizers instrument the host side only.
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-std=c++17", "-fPIC",
                           "-shared", "-Xarch_host", "-g",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                           "-Xarch_host", "-fno-sanitize-recover=all",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-I", os.path.join(ROOT, "include"), "-o", str(lib), *srcs],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    _run_tests({"LD_PRELOAD": asan[0], "PAGEDATTN_LIB": str(lib)}, ["tests/test_abi.py"], tmp_path)
