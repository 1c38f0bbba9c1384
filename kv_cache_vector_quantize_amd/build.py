"""In-tree build of libtq.so (hipcc, gfx950).

``python -m kv_cache_vector_quantize_amd.build`` compiles every source under
``csrc/`` into an object file (in parallel) and links
``kv_cache_vector_quantize_amd/libtq.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops stay off for correctness (see design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
]


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# Host sources rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer
# (host pass only: each -fsanitize follows -Xarch_host, the device code of
# the kernels is unchanged) and linked with the regular kernel objects.
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libtq_san.so")
SAN_HOST_SOURCES = ("codebook_host.cpp", "tq_api.cpp")
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-g",
]


def sanitizer_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (it also carries the
    UndefinedBehaviorSanitizer handlers), to be preloaded into a host process."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "llvm")
    r = subprocess.run([os.path.join(llvm, "bin", "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang's AddressSanitizer runtime was not found")
    return path


def build_sanitized(verbose: bool = False) -> str:
    """libtq_san.so: the regular kernel objects with sanitized host sources
    (the regular build must exist, or is made first)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    for src in _sources():
        if src in SAN_HOST_SOURCES:
            obj = os.path.join(SAN_DIR, src + ".o")
            cmd = [HIPCC, "-xhip", *COMMON, *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        else:
            obj = os.path.join(BUILD, src + ".o")
            if not os.path.exists(obj):
                obj = _compile(src)
        objs.append(obj)
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
