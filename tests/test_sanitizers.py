"""Host-side sanitizer runs (no GPU): the fp64 oracle built with
AddressSanitizer + UndefinedBehaviorSanitizer runs its pins and the parity
harness's CPU checks, and the library built with AddressSanitizer on its host
code (argument checks, workspace planning, the C ABI) runs the boundary
tests.  Each run is a subprocess with the sanitizer runtime preloaded; any
report aborts it."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _gcc_asan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run_pytest(env_extra, files):
    env = dict(os.environ)
    env.update(env_extra)
    env.update(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", *files]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    return tail


def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    asan = _gcc_asan()
    if asan is None:
        pytest.skip("gcc's libasan is not installed")
    from oracle import build
    lib = build.build(out=str(tmp_path / "liboracle_hikvp_san.so"), sanitize=True)
    out = _run_pytest({"LD_PRELOAD": asan, "HIKVP_ORACLE_LIB": lib},
                      ["tests/test_oracle_pins.py", "tests/test_parity_harness.py"])
    assert " passed" in out


def test_library_host_code_under_address_sanitizer(tmp_path):
    asan = _clang_asan()
    if asan is None:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    from hierarchical_kv_pruning_amd import build
    # host-only instrumentation: each sanitizer flag applies to the host pass
    flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    lib = build.build(out=str(tmp_path / "libatlaskv_asan.so"), extra_flags=flags)
    out = _run_pytest({"LD_PRELOAD": asan, "ATLASKV_LIB": lib}, ["tests/test_boundary.py"])
    assert " passed" in out
