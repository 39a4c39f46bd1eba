"""The C shim's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

build.py's host-sanitizer variant compiles the host code with both sanitizers
(the kernels as in the release build) and with the debug range checks; this test runs
tests/test_abi_host.py against it in a subprocess with the sanitizer runtime
preloaded, and fails on any sanitizer report.  CPU only."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _clang_rt() -> str:
    clang = "/opt/rocm/lib/llvm/bin/clang"
    r = subprocess.run([clang, "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    assert r.returncode == 0 and os.path.isabs(path) and os.path.exists(path), r.stdout + r.stderr
    return path


def test_abi_host_checks_under_asan_and_ubsan():
    from head_latent_attention_kv_amd import build
    lib = build.lib_path("hostsan")
    if not os.path.exists(lib):
        build.build(variant="hostsan")
    env = dict(os.environ, LD_PRELOAD=_clang_rt(), MLA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:detect_odr_violation=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout
