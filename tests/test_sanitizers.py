"""CPU sanitizer runs: the oracle (plain C) built with AddressSanitizer and
UndefinedBehaviorSanitizer runs the oracle's own pin tests, and liblk.so with its host
code instrumented the same way runs the C-ABI validation tests (no kernel is launched
there).  Any sanitizer report aborts the child run and fails the test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_TESTS = ["tests/test_oracle.py", "tests/test_oracle_rope.py", "tests/test_oracle_mla.py"]
ASAN_OPTIONS = "detect_leaks=0:alloc_dealloc_mismatch=0:new_delete_type_mismatch=0:abort_on_error=1"


def _run_child(env_extra, tests):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = ASAN_OPTIONS
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"sanitized run failed (rc {r.returncode}):\n{tail}"
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    return tail


def test_oracle_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    from oracle import oracle as O
    lib = O.build_sanitized(str(tmp_path / "liblk_oracle_san.so"))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's libasan runtime not found")
    out = _run_child({"LK_ORACLE_LIB": lib, "LD_PRELOAD": asan}, ORACLE_TESTS)
    assert "passed" in out


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not os.path.exists(hipcc) or not rts:
        pytest.skip("hipcc or clang's ASan runtime not available")
    from sparse_attention_lightning_fp8_amd import build as B
    lib = B.build_host_sanitized(str(tmp_path / "san"))
    out = _run_child({"LK_LIB_PATH": lib, "LD_PRELOAD": rts[0]}, ["tests/test_abi.py"])
    assert "passed" in out
