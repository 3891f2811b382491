"""Host-side sanitizer build of libveda: AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (the plan, the budgets, the
argument checks and the C ABI), the GPU code compiled as usual.  For CPU
tests: the host plan tests run against it (tests/test_host_sanitized.py).

    python -m block_sparse_attention_10_amd.build_sanitized     # prints the path

The library goes to _build/ at the repository root (not loaded by the
package); a process that loads it must preload the sanitizer runtime
(asan_runtime() names it).
"""

import glob
import os
import subprocess
import sys

from . import build as b

OUT_DIR = os.path.join(b.ROOT, "_build")
LIB = os.path.join(OUT_DIR, "libveda_host_sanitized.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that matches hipcc's host compiler."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(b.hipcc())))
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under " + rocm)
    return hits[-1]


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [b.hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # sanitizers on the host pass only
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-shared-libasan",
           "-I", b.INCLUDE, "-I", b.CSRC]
    cmd += [os.path.join(b.CSRC, s) for s in b.SOURCES]
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("sanitized libveda build failed:\n" + out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
