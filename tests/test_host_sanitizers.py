"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with -fsanitize=address,undefined on its host code only (the
device code is compiled as usual; every call below is rejected, or answered, by the host
code before any HIP call), and the host-side ABI tests run against that build in a child
process with the sanitizer runtime preloaded.  Any report fails the test."""
import os
import subprocess
import sys

import pytest

from long_context_attention_polar_amd import build as pbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime(hipcc):
    res = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_checks_under_host_sanitizers(tmp_path):
    hipcc = pbuild.hipcc()
    runtime = _asan_runtime(hipcc)
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    lib = tmp_path / "libpolar_attn_host_sanitized.so"
    sanitize = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libasan",
                "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [hipcc, f"--offload-arch={pbuild.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           *pbuild.HIP_FLAGS, *sanitize, "-I", os.path.join(ROOT, "include"),
           os.path.join(pbuild.CSRC, "polar_attn.hip"), "-o", str(lib)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ)
    log = tmp_path / "sanitizer"
    env.update(POLAR_TEST_LIB=str(lib), LD_PRELOAD=runtime,
               ASAN_OPTIONS=f"detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:halt_on_error=1:"
                            f"log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi.py"),
                          "-k", "not exports_every_declared and not build_compiles"],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    logs = "".join(p.read_text()[:3000] for p in tmp_path.glob("sanitizer*"))
    report = run.stdout[-3000:] + run.stderr[-3000:] + logs
    assert run.returncode == 0 and not logs, report
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert " passed" in run.stdout, report
