"""The C ABI layer (abi.cpp) built with AddressSanitizer on the host pass and
driven through every validation path on the CPU (tests/asan_abi_driver.py).
The sanitizer runtime is preloaded into a fresh interpreter that imports
neither torch nor the package; a heap or stack error ends it with the
sanitizer's report and a non-zero status."""

import os
import subprocess
import sys

import pytest

from selective_state_space_mamba3_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_layer_is_clean_under_address_sanitizer():
    try:
        lib = build.build_asan()
        runtime = build.asan_runtime()
    except RuntimeError as e:  # pragma: no cover - toolchain without the sanitizer runtime
        pytest.skip(str(e))
    env = dict(os.environ, LD_PRELOAD=runtime, HIP_VISIBLE_DEVICES="-1",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=23:detect_stack_use_after_return=1")
    res = subprocess.run([sys.executable, os.path.join(HERE, "asan_abi_driver.py"), lib], env=env, cwd=HERE,
                         capture_output=True, text=True, timeout=300)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert "asan driver:" in res.stdout
