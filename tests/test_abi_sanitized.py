"""The C ABI's argument validation under host AddressSanitizer + UBSan (CPU only).

The library is rebuilt with every host pass instrumented (the gfx950 code as
usual), and the argument-checking tests of test_abi.py run against it in a
child process that preloads the ASan runtime: an out-of-bounds access, a use
after free, a signed overflow or a misaligned access in the validation,
workspace-layout or error-reporting code aborts the child.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
import ctypes
assert hasattr(ctypes.CDLL(None), "__asan_init"), "the ASan runtime is not loaded"
import fp4_quantized_rl_amd as fr
fr.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {abi!r}, "-m", "not gpu",
                      "-k", "not valid_call_without_gpu and not binding_fails_loudly"]))
"""


def test_validation_layer_is_clean_under_asan_and_ubsan():
    from fp4_quantized_rl_amd import build as b
    try:
        runtime = b.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = b.build_sanitized()
    # the host code really is instrumented: the library imports the sanitizers' checks
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in undef and "__ubsan_handle" in undef
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime + ((" " + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                        abi=os.path.join(ROOT, "tests", "test_abi.py"))
    res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in res.stdout, out[-2000:]
