"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer, with the DLLM_DEBUG internal checks on: a build
of the library whose host code is instrumented (the device code is built as
usual and never runs here) runs the ABI and binding-check suites, whose
cases exercise argument validation, workspace carving and the error paths
before any HIP call, and the no-device error path."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "masked_token_logits_amd", "csrc")
sys.path.insert(0, ROOT)
from masked_token_logits_amd.build import SOURCES  # noqa: E402  (the library's own source list)


def _asan_runtime(hipcc):
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(c):
            r = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
            p = r.stdout.strip()
            if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
                return p
    return None


def test_abi_suites_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    rt = _asan_runtime(hipcc)
    if rt is None:
        pytest.skip("ASan runtime not found")
    lib = str(tmp_path / "libdllm_readout_asan.so")
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-shared",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-DDLLM_DEBUG",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC] + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, DLLM_TEST_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", "test_abi_cpu.py"), os.path.join(ROOT, "tests", "test_binding_checks_cpu.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
