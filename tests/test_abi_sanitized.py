"""The host-side ABI checks of test_abi.py, run against a build of the
library whose host code (argument validation, workspace planning, launch
set-up) carries AddressSanitizer and UndefinedBehaviorSanitizer. They run in
a child process that preloads clang's ASan runtime; any report (an
out-of-bounds access, a use after free, an overflow in the planning
arithmetic) makes the child fail. No device code runs: every call is
rejected before its first HIP call, as in test_abi.py."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_are_clean_under_asan_and_ubsan():
    from long_context_kv_snapkv_amd.build import asan_runtime, build_sanitized

    try:
        lib = build_sanitized()
        runtime = asan_runtime()
    except RuntimeError as e:  # no ROCm toolchain here
        pytest.skip(str(e))
    # the host code is instrumented (it calls the sanitizers' report hooks)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    if nm.returncode == 0:
        assert "__asan_report" in nm.stdout and "__ubsan_handle" in nm.stdout
    code = ("import sys; sys.path.insert(0, {root!r}); "
            "from long_context_kv_snapkv_amd import snapkv; snapkv.LIB_PATH = {lib!r}; "
            "import pytest; "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            "{tests!r}]))").format(root=ROOT, lib=lib,
                                   tests=os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
