"""Build libgt_attn.so in-tree for gfx950 with hipcc (no GPU needed to compile).

    python -m graph_transformer_attention_amd.build             # or build() from Python
    python -m graph_transformer_attention_amd.build --sanitize  # libgt_attn_san.so, host checks

The --sanitize variant builds the host code of every source (argument checks, workspace
sizing, the breadth-first distance-code builder, launch set-up) with AddressSanitizer
and UndefinedBehaviorSanitizer; device code is compiled as usual. It is for CPU runs of
the host tests: load it in place of the product library with GT_ATTN_LIBRARY and
preload the sanitizer runtime that SANITIZER_RUNTIME names (the Python interpreter is
not instrumented itself).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgt_attn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 arithmetic is switched off for every HIP file.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics", "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]

SAN_LIB = os.path.join(PKG, "libgt_attn_san.so")
SAN_OBJ = os.path.join(PKG, "_build_san")
# Host-side only: each sanitizer flag is bound to the host compilation.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]
SAN_LINK = ["-shared-libasan", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
SANITIZER_RUNTIME = "libclang_rt.asan-x86_64.so"


def _sources():
    out = []
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip") or f.endswith(".cpp"):
            out.append(os.path.join(CSRC, f))
    return out


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_OBJ if sanitize else OBJ, os.path.basename(src) + ".o")
    extra = SAN_FLAGS if sanitize else []
    if src.endswith(".hip"):
        cmd = [HIPCC, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, "-x", "c++", *CXX_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(SAN_OBJ if sanitize else OBJ, exist_ok=True)
    srcs = _sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), srcs))
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *(SAN_LINK if sanitize else []), *objs,
           "-o", tmp, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime the --sanitize library links against."""
    r = subprocess.run([HIPCC, f"-print-file-name={SANITIZER_RUNTIME}"], capture_output=True, text=True)
    return r.stdout.strip()


if __name__ == "__main__":
    if "--runtime" in sys.argv:
        print(sanitizer_runtime())
    else:
        build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)
