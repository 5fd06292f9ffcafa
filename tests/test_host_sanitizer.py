"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host_sanitizer/build_host_san.py compiles every library source for the
host only, with -fsanitize=address,undefined (recoverable UB made fatal), and
links it against stubs of the HIP runtime whose device calls all fail.  This
test runs the host ABI tests (tests/test_abi.py and the host test of the
no-allocation entry point) plus dispatch checks that drive every entry point
past validation into the split planning and the (stubbed) launches, in a
subprocess that preloads the ASan runtime and loads that build through
ATTN_LIB_PATH.  Any sanitizer report aborts the subprocess and fails here.
"""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_runs_clean_under_asan_and_ubsan():
    sys.path.insert(0, os.path.join(ROOT, "tests", "host_sanitizer"))
    import build_host_san
    lib = build_host_san.build()
    env = dict(os.environ)
    env.update({
        "ATTN_LIB_PATH": lib,
        "ATTN_HOST_SANITIZER": "1",
        "LD_PRELOAD": build_host_san.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    cmd = [sys.executable, "-m", "pytest", "-v", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not gfx950_build",
           os.path.join(ROOT, "tests", "test_abi.py"),
           os.path.join(ROOT, "tests", "test_zz_no_alloc.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout, res.stdout[-2000:]
    # The dispatch checks ran (they are skipped against any other build).
    assert "test_dispatch_variants PASSED" in res.stdout, res.stdout[-2000:]
    assert res.stdout.count("test_dispatch_attn_fwd[") >= 7, res.stdout[-2000:]
    assert "SKIPPED" not in res.stdout, res.stdout[-2000:]
