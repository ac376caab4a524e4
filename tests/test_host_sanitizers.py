"""The library's host code (api.cpp: argument checks, batch assembly, tile
planning, the graph cache) under AddressSanitizer and
UndefinedBehaviorSanitizer.

``libsnrvq_hostsan.so`` is the same library with api.cpp built with host
ASan + UBSan (no sanitizer in device code).  The host-only ABI tests run
again against it in a child process with the compiler's ASan runtime
preloaded; any invalid access or undefined behaviour aborts the child.  The
same environment (``sanitizer_env()``) runs the GPU tests on a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from streaming_neural_audio_rvq_amd import _build  # noqa: E402


def sanitizer_env() -> dict:
    """Environment of a process that loads the host-sanitized library: the
    ASan runtime first among the preloads (any preload already set stays),
    leaks not reported (the interpreter's own allocations), the first error
    fatal."""
    if not os.path.exists(_build.LIB_HOSTSAN):
        raise FileNotFoundError(f"{_build.LIB_HOSTSAN} is missing: build it first "
                                "(python -c 'import __graft_entry__ as g; g.build()')")
    env = dict(os.environ)
    pre = [_build.asan_runtime()] + [p for p in env.get("LD_PRELOAD", "").split(":") if p]
    env["LD_PRELOAD"] = ":".join(pre)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["SNRVQ_LIBRARY"] = _build.LIB_HOSTSAN
    return env


def run_child(args, timeout=600):
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=sanitizer_env(),
                       capture_output=True, text=True, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def test_child_runs_the_instrumented_library_with_asan_active():
    code = ("import ctypes, streaming_neural_audio_rvq_amd as snr\n"
            "L = snr.lib()\n"
            "assert snr.LIB_PATH.endswith('libsnrvq_hostsan.so'), snr.LIB_PATH\n"
            "ctypes.CDLL(None).__asan_address_is_poisoned\n"  # the runtime is in the process
            "print('ok', snr.chunk_plan(20, (1, 2, 4), 8))\n")
    rc, out = run_child(["-c", code], timeout=120)
    assert rc == 0, out
    assert "ok [1, 2, 4, 8, 5]" in out, out
    syms = subprocess.run(["nm", "-D", _build.LIB_HOSTSAN], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms


@pytest.mark.timeout(900)
def test_host_abi_tests_pass_under_asan_and_ubsan():
    rc, out = run_child(["-m", "pytest", "tests/test_host_abi.py", "-q", "-x",
                         "-p", "no:cacheprovider"])
    assert rc == 0, out[-4000:]
    assert "passed" in out and "AddressSanitizer" not in out and "runtime error" not in out, \
        out[-4000:]
