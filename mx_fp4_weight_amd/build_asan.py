"""Host-sanitizer build of the C-ABI layer, for the CPU checks of its argument validation.

api.hip (the entry points: argument checks, topology building, dispatch) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer on its HOST code only (device code is built as
usual) and linked with the
regular objects of the kernel files into <repo>/_build/asan/libmxfp4spec.so. Run
tests/test_abi_cpu.py against it with MXS_LIB pointing there and the clang ASan runtime
preloaded (tests/test_abi_asan.py does both).
"""
from __future__ import annotations

import glob
import os
import subprocess

from mx_fp4_weight_amd import build as b

OUT_DIR = os.path.join(b.BUILD, "asan")
LIB = os.path.join(OUT_DIR, "libmxfp4spec.so")
# AddressSanitizer and UndefinedBehaviorSanitizer (shifts past the width, overflow, bad
# alignment, ... abort the process) on the host code only.
HOST_ASAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
             "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()


def asan_runtime() -> str | None:
    """The clang ASan runtime shipped with the ROCm LLVM (preloaded into an uninstrumented python)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")) + \
        sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"))
    return hits[-1] if hits else None


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src in b.SOURCES:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        extra = HOST_ASAN if src == "api.hip" else []
        cmd = [b.HIPCC, *b.FLAGS, *b.SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(b.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        objs.append(obj)
    cmd = [b.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_ASAN[:4], *objs, "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
