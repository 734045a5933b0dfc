"""Build libdit_block with AddressSanitizer and UndefinedBehaviorSanitizer
in its host code (argument checks, workspace layout, stack bookkeeping),
for the CPU ABI tests; the device code is built as usual.

Usage: python -m diffusion_transformer_dit_amd.build_sanitized
Output: _build/asan/libdit_block.so (load it with DIT_LIB=<path> and the
clang ASan runtime preloaded, see tests/test_abi_sanitized.py).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from diffusion_transformer_dit_amd.build import ARCH, COMMON_FLAGS, CSRC, INCLUDE, ROOT, hipcc

OUT_DIR = os.path.join(ROOT, "_build", "asan")
LIB_PATH = os.path.join(OUT_DIR, "libdit_block.so")
# every sanitizer flag applies to the host pass only
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else ""


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *HOST_SANITIZE, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SANITIZE, "-o", LIB_PATH, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return LIB_PATH


if __name__ == "__main__":
    print(build())
    sys.exit(0)
