"""bench.py command line: the multi-GPU request is refused before any device work."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "--gpus 2" in res.stderr
    assert res.stdout == ""   # no JSON line is printed


def test_kernel_code_hash_of_the_built_library():
    """The hash that keeps recorded traffic valid is taken from the attention
    kernel's machine code in the built library: present for both head
    dimensions, 16 hex digits, different between them, and stable across
    calls."""
    import pytest
    sys.path.insert(0, ROOT)
    import bench
    lib = os.path.join(ROOT, "block_sparse_attention_10_amd", "libveda.so")
    if not os.path.exists(lib):
        pytest.skip("library not built")
    h128, h64 = bench.kernel_code_sha(lib, 128), bench.kernel_code_sha(lib, 64)
    for h in (h128, h64):
        assert len(h) == 16 and int(h, 16) >= 0
    assert h128 != h64
    assert bench.kernel_code_sha(lib, 128) == h128
