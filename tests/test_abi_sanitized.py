"""The host-side ABI tests (argument validation, size queries, error
strings, the binding's buffer checks) against a build of the library whose
host code runs under AddressSanitizer and UndefinedBehaviorSanitizer.

The sanitised library is built by ``taylor_recurrent_states_amd.build``'s
``build_sanitized`` (device code as usual, cached until a source changes) and
loaded through ``TT_LIBRARY`` in a child process that has clang's ASan
runtime preloaded.  No kernel is launched: the child runs only tests that
need no GPU.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_checks_under_host_sanitizers(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's ASan runtime is not installed")
    from taylor_recurrent_states_amd import build
    lib = build.build_sanitized()
    log = tmp_path / "san"
    env = dict(os.environ)
    env.update({
        "TT_LIBRARY": lib,
        "LD_PRELOAD": rt,
        # Python and torch themselves are not instrumented: no leak check,
        # no allocator-pairing or ODR checks across their libraries
        "ASAN_OPTIONS": f"detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:halt_on_error=1:"
                        f"log_path={log}",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={log}",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "tests/test_binding_checks.py", "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(f"{log}*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-3000:] + reports[-4000:])
    assert " passed" in r.stdout
