"""The CPU code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

1. The oracle, built with both sanitizers, runs every oracle pin.
2. The library's host code (argument validation, workspace sizing, dispatch up
   to the first launch), built with both sanitizers on the host side only,
   runs the C-ABI tests, which force every validation error.
Each run is a child process with the sanitizer runtime preloaded; any report
ends it with a non-zero status (UBSan reports are made fatal)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV_SAN = {
    "ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:abort_on_error=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _run_pytest(test_file, extra_env):
    env = dict(os.environ, **ENV_SAN, **extra_env)
    # -s: a sanitizer report goes straight to the output instead of a capture file
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", test_file)], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out


def test_oracle_pins_under_sanitizers(tmp_path):
    from oracle import build as ob
    lib = ob.build_sanitized(str(tmp_path))
    _run_pytest("test_oracle_pins.py", {"SQ_ORACLE_LIB": lib, "LD_PRELOAD": ob.asan_runtime()})


def test_abi_validation_under_sanitizers(tmp_path):
    import importlib.util
    spec = importlib.util.spec_from_file_location("_sq_build", os.path.join(ROOT, "int8_quantization_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    try:
        rt = b.host_asan_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    lib = b.build_host_sanitized(str(tmp_path))
    _run_pytest("test_abi_cpu.py", {"SQ_LIB": lib, "LD_PRELOAD": rt})
