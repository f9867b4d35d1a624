"""The host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

`dequant_gemv_amd.build.build_sanitized()` instruments the host pass of dqg_api.cpp (argument
validation, workspace layout and size queries, plan selection); this test runs every case of
test_abi_cpu.py against that build in a child process with the ASan runtime preloaded.  No
GPU is touched: every call there fails validation before a launch."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_are_clean_under_host_sanitizers():
    from dequant_gemv_amd import build as bld
    try:
        runtime = bld.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = bld.build_sanitized(verbose=False)
    env = dict(os.environ)
    env["DQG_LIBRARY"] = lib
    env["LD_PRELOAD"] = ":".join(p for p in (runtime, os.environ.get("LD_PRELOAD", "")) if p)
    # the interpreter and torch are not instrumented: leaks at exit are theirs
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = ("import sys, pytest\n"
            "from dequant_gemv_amd import binding as B\n"
            f"assert B.LIB_PATH == {lib!r}, B.LIB_PATH\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', "
            f"{os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
