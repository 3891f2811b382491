"""The host plan tests (tests/test_host_plan.py: plan creation against the
oracle, budgets, validation errors, host checks before any launch, plans and
errors from several threads) run against a build of libveda whose host code
carries AddressSanitizer and UndefinedBehaviorSanitizer; any report fails the
run.  CPU only: the library's GPU code is built but never launched here."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow

if not (os.environ.get("HIPCC") or shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
    pytest.skip("hipcc not available", allow_module_level=True)

_RUNNER = """
import sys
sys.path.insert(0, %(root)r)
sys.path.insert(0, %(tests)r)
from block_sparse_attention_10_amd import binding as vb
vb.LIB_PATH = %(lib)r            # the sanitized build instead of the in-tree one
import pytest
rc = pytest.main([%(test)r, "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"])
assert vb.loaded_library() == %(lib)r, vb.loaded_library()
sys.exit(int(rc))
"""


def test_host_plan_tests_pass_under_asan_and_ubsan():
    from block_sparse_attention_10_amd import build_sanitized as bs
    lib = bs.build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = bs.asan_runtime()
    # CPython's own allocations are not freed at exit: leak reports are off;
    # every other AddressSanitizer or UBSan report aborts the run
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = _RUNNER % {"root": ROOT, "tests": os.path.join(ROOT, "tests"), "lib": os.path.realpath(lib),
                      "test": os.path.join(ROOT, "tests", "test_host_plan.py")}
    res = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=600)
    tail = "\n".join(res.stdout.splitlines()[-40:])
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in res.stdout and "runtime error:" not in res.stdout, tail
    assert " passed" in res.stdout, tail
