"""CPU sanitizer checks (no GPU is used):

  * the oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer:
    the oracle tests run in a child process with the ASan runtime preloaded
    and ORACLE_LIB naming the sanitized build;
  * libgradcomp's host code (plan validation and layout, message and
    workspace sizes, every entry point's argument checks) under both
    sanitizers and LeakSanitizer, driven by a C program (abi_host_checks.c),
    with the device code built as in the product.

Any report from a sanitizer ends the child with a non-zero status."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from tests import sanitize_build as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_suite_under_asan_and_ubsan(tmp_path):
    lib = S.build_oracle(str(tmp_path))
    env = dict(os.environ, LD_PRELOAD=S.gcc_runtime("libasan.so"), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", ORACLE_LIB=lib)
    # the child loads the sanitized build, not the product one
    r = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.lib()._name)"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stdout + r.stderr
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    assert tests
    r = subprocess.run([sys.executable, "-m", "pytest", *tests, "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout


@pytest.mark.skipif(not (os.path.exists(S.CLANG) and os.path.exists(S.hip_build.HIPCC)),
                    reason="needs the ROCm toolchain")
def test_host_entry_points_under_asan_ubsan_and_lsan(tmp_path):
    S.build_host_library(str(tmp_path))
    exe = S.build_driver(str(tmp_path), str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok")
