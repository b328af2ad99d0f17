"""Host code under the compiler sanitizers (CPU only).

  * The C-ABI validation layer (api.cpp with shapes.cpp), built for the host
    alone with g++ over a stub of the three HIP runtime calls it makes and of
    the kernel launchers (tests/sanitize/hip_stub.cpp), runs the driver
    tests/sanitize/abi_host_check.cpp under AddressSanitizer +
    UndefinedBehaviorSanitizer and, separately, ThreadSanitizer.
  * The oracle (oracle/oracle.c) runs its worker-pool driver
    tests/sanitize/oracle_threads.c under ThreadSanitizer and under
    AddressSanitizer + UndefinedBehaviorSanitizer, and the whole oracle pin
    suite (tests/test_oracle_pins.py) runs against an ASan/UBSan build of it.

No GPU code is built here: every build below is gcc/g++ on host sources.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "differential_attention_prefill_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")

ASAN_UBSAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
TSAN = ["-fsanitize=thread"]
ENV_RUN = {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
           "TSAN_OPTIONS": "halt_on_error=1:second_deadlock_stack=1"}


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc/g++ not available")
    if not _runtime("libasan.so") or not _runtime("libtsan.so") or not _runtime("libubsan.so"):
        pytest.skip("sanitizer runtimes not installed")
    return str(tmp_path_factory.mktemp("sanitize"))


def _build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, "build failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-4000:])


def _run(exe, extra_env=None):
    env = dict(os.environ)
    env.update(ENV_RUN)
    env.update(extra_env or {})
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, "%s failed (%d):\n%s\n%s" % (exe, r.returncode, r.stdout[-3000:],
                                                          r.stderr[-6000:])
    return r.stdout


def _abi_build(outdir, flags, name):
    exe = os.path.join(outdir, name)
    _build(["g++", "-std=c++17", "-g", "-O1", "-Wall", "-Werror"] + flags +
           ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
            "-I" + CSRC, "-I" + SAN, os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "shapes.cpp"),
            os.path.join(SAN, "hip_stub.cpp"), os.path.join(SAN, "abi_host_check.cpp"), "-pthread",
            "-o", exe])
    return exe


def test_abi_validation_under_asan_ubsan(outdir):
    out = _run(_abi_build(outdir, ASAN_UBSAN, "abi_asan"))
    assert "0 failed" in out


def test_abi_validation_under_tsan(outdir):
    out = _run(_abi_build(outdir, TSAN, "abi_tsan"))
    assert "0 failed" in out


@pytest.mark.parametrize("flags,name", [(TSAN, "oracle_tsan"), (ASAN_UBSAN, "oracle_asan")])
def test_oracle_pool_under_sanitizer(outdir, flags, name):
    exe = os.path.join(outdir, name)
    _build(["gcc", "-std=c11", "-g", "-O1", "-Wall", "-Werror"] + flags +
           ["-pthread", ORACLE_C, os.path.join(SAN, "oracle_threads.c"), "-o", exe, "-lm"])
    out = _run(exe)
    assert "0 failures" in out


def test_oracle_pins_under_asan_ubsan(outdir):
    lib = os.path.join(outdir, "liboracle_asan.so")
    _build(["gcc", "-std=c11", "-g", "-O1", "-Wall"] + ASAN_UBSAN +
           ["-fPIC", "-shared", "-pthread", ORACLE_C, "-o", lib, "-lm"])
    env = dict(os.environ)
    env.update(ENV_RUN)
    # The interpreter is not instrumented: its own allocations are not leak-checked.
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["LD_PRELOAD"] = _runtime("libasan.so") + ":" + _runtime("libubsan.so")
    env["DIFFATTN_ORACLE_LIB"] = lib
    code = ("import oracle, sys; assert oracle._LIB_PATH == %r, oracle._LIB_PATH; "
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))"
            % (lib, os.path.join(ROOT, "tests", "test_oracle_pins.py")))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
