"""Build librma_san.so: the same sources with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only (argument checks, sizes, launch
set-up).  Device code is compiled as usual; GPU sanitizers are not used.

The library goes to a fresh temporary directory (``build_sanitized()`` returns its
path; the caller removes it); it needs the clang ASan runtime preloaded into an
uninstrumented interpreter (``asan_runtime()`` gives its path).  It is a test
build: nothing in the package loads it, and none of it stays in the tree.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import tempfile

from .build import ARCH, CSRC, INCLUDE, _hipcc, sources
SAN_FLAGS = [
    f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SAN_LINK = [
    f"--offload-arch={ARCH}", "-shared", "-fPIC",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-shared-libsan",
]


def asan_runtime() -> str:
    """Path of the clang ASan runtime that the sanitized library links against."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "bin",
                         "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def _compile(src: str, out_dir: str) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *SAN_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_sanitized() -> str:
    """Build into a new temporary directory; returns the library's path."""
    out_dir = tempfile.mkdtemp(prefix="librma_san_")
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir), srcs))
    lib = os.path.join(out_dir, "librma_san.so")
    cmd = [_hipcc(), *SAN_LINK, *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build_sanitized())
