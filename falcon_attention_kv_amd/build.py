"""Builds libunipin.so (the C-ABI library and its gfx950 kernels) in place with hipcc.

Usage: python falcon_attention_kv_amd/build.py   (or call build()).  It runs as a plain
script: importing the package first would load the library it is about to replace.
Always recompiles; the result is falcon_attention_kv_amd/libunipin.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libunipin.so")
# measurement probes (matrix-core peak, matrix/vector overlap): their own library, loaded
# only by the benchmark
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB = os.path.join(PKG, "libunipin_probe.so")
SOURCES = ["unipin.cpp", "pool_share.cpp", "pool_status.hip", "attn_bf16.hip", "attn_fp32.hip", "attn_ar.hip",
           "block.cpp", "block_kernels.hip", "gemm_bf16.hip"]
# hipBLASLt is one of the two GEMM kernel families of the block; found at run time through
# the ROCm library path.  librt: the shared pages of pools shared between processes.
LINK = ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib", "-lrt"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (needs ROCm)")


def common_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
            # packed fp32 VALU instructions stay off in every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, extra, verbose: bool) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + common_flags() + list(extra)
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out, link, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs + link
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


# Host sources (no device code): the ones the sanitized host build instruments.
HOST_SOURCES = [s for s in SOURCES if s.endswith(".cpp")]
SANITIZED_DIR = os.path.join(OUT_DIR, "sanitized")
SANITIZED_LIB = os.path.join(SANITIZED_DIR, "libunipin_host_sanitized.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host side only (-Xarch_host before
# each option); the kernels are the ordinary objects of build().
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-shared-libasan", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (preloaded into the process
    that loads the sanitized library)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found")
    return path


def build_host_sanitized(verbose: bool = False) -> str:
    """libunipin with its host code (descriptors, checks, dispatch, sharing, the block's
    plans) built with AddressSanitizer and UndefinedBehaviorSanitizer, linked against the
    kernel objects of the last build().  For CPU tests of the host paths; never loaded
    by the package."""
    os.makedirs(SANITIZED_DIR, exist_ok=True)
    kernels = [os.path.join(OUT_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES if s.endswith(".hip")]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        raise RuntimeError(f"run build() first (missing {missing[0]})")

    def compile_host(src: str) -> str:
        obj = os.path.join(SANITIZED_DIR, os.path.splitext(src)[0] + ".o")
        flags = [f for f in common_flags() if f != "-O3"]
        cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + flags + ["-O1", "-g", "-fno-omit-frame-pointer"]
        cmd += SANITIZE
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(HOST_SOURCES)) as ex:
        objs = list(ex.map(compile_host, HOST_SOURCES))
    _link(objs + kernels, SANITIZED_LIB, LINK + SANITIZE, verbose)
    return SANITIZED_LIB


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, LINK, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, [], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
