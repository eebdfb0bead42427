"""The C ABI's validation layer under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

api.cpp and plan.cpp are built for the CPU with both sanitizers and linked
against stub kernel launchers (tests/sanitize/), and tests/test_abi.py runs
again in a child process that loads that library instead of the real one,
with the sanitizer runtimes preloaded.  Every argument check, workspace
computation and size limit then runs instrumented, and the calls that pass
validation run as far as their (stub) launch.  A second child reads one past
the end of a heap array through the same library, to show that the runtime
is live there: it must stop with a heap-buffer-overflow report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "tests", "sanitize"))
import build_validation_lib as V  # noqa: E402


@pytest.fixture(scope="module")
def san_env():
    try:
        lib = V.build()
        pre = V.runtime_preload()
    except (RuntimeError, FileNotFoundError) as e:
        pytest.skip(f"sanitizer toolchain unavailable: {e}")
    env = dict(os.environ)
    # the sanitizer runtimes must be the first preloaded libraries
    env["LD_PRELOAD"] = pre + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["ATTN_VALIDATION_LIB"] = lib
    return env


def test_abi_cases_run_clean_under_sanitizers(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=san_env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    tail = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in r.stdout and "skipped" not in r.stdout, tail  # the stub-only cases ran too


def test_sanitizer_is_live_in_the_child(san_env):
    code = ("import ctypes, os; L = ctypes.CDLL(os.environ['ATTN_VALIDATION_LIB']); "
            "assert L.attn_stub_heap_read(4, 3) == 4; print('in bounds ok', flush=True); L.attn_stub_heap_read(4, 4)")
    r = subprocess.run([sys.executable, "-c", code], env=san_env, cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert "in bounds ok" in r.stdout
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
