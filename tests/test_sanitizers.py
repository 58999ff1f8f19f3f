"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: both are rebuilt with the sanitizers (the
library's device code is the normal gfx950 build; only its host side --
argument checks, workspace layout, launch planning -- is instrumented) and
the oracle's pinned tests and the C-ABI tests run against those builds in a
child process with the sanitizer runtime preloaded. Any report fails the
run (UBSan does not recover; ASan stops at its first error)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = "/opt/rocm/lib/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"

# the oracle tests that exercise every oracle entry point on small cases, and
# the host-side library tests
TESTS = ["tests/test_oracle_philox_tree.py", "tests/test_oracle_attention.py", "tests/test_oracle_paged.py",
         "tests/test_oracle_fp8.py", "tests/test_oracle_sampler.py", "tests/test_oracle_min_p.py",
         "tests/test_oracle_truncation.py", "tests/test_oracle_allowed_set.py", "tests/test_oracle_lossy.py",
         "tests/test_oracle_deterministic.py", "tests/test_oracle_pack.py", "tests/test_abi.py"]


@pytest.mark.skipif(not os.path.exists(ASAN_RT), reason="the ROCm LLVM AddressSanitizer runtime is not installed")
def test_oracle_and_host_code_under_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle.build_oracle import build_oracle_sanitized
    from sanitize_build import build_host_sanitized

    oracle_so = build_oracle_sanitized(str(tmp_path / "liboracle_san.so"))
    lib_so = build_host_sanitized(str(tmp_path / "libspecverify_san.so"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = ASAN_RT
    # leaks: the interpreter and torch keep allocations alive at exit by design;
    # alloc/dealloc mismatches: reported inside uninstrumented libraries too
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:verify_asan_link_order=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize_run.py"), oracle_so, lib_so,
                          "-x", "-q", "-m", "not gpu", *TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=1500)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error:" not in res.stderr, tail
    assert " passed" in res.stdout, tail
