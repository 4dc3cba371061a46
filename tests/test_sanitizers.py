"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the
oracle's pins (tests/test_oracle_pins.py) run again in a child process
against an instrumented build of oracle.c (gcc -fsanitize=address,undefined,
errors fatal), with gcc's ASan runtime preloaded.  Any out-of-bounds
access, use after free or undefined behaviour in the oracle fails the run.
Leak checking is off: the Python interpreter's own allocations would
report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        p = subprocess.run(["gcc", "-print-file-name=%s" % name], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_oracle_pins_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    import oracle.binding as ob
    ob.build_oracle(force=False, sanitize=True)
    env = dict(os.environ, ORACLE_SANITIZED="1", LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out


def test_capi_host_paths_under_asan_and_ubsan():
    """The C ABI layer's host paths (validation, workspace sizes, the rotary
    table, status strings) under AddressSanitizer and UBSan: capi.cpp is
    rebuilt with host-only sanitizers and the host ABI tests run against it
    in a child process (no GPU call is made)."""
    sys.path.insert(0, ROOT)
    from learned_sparse_causal_amd import build
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    try:
        lib = build.build_sanitized_host()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    env = dict(os.environ, MONO_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_capi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
