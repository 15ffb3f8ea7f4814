"""Build librelattn.so for gfx950 in-tree.

    python -m relative_position_encoding_amd.build

Compiles the HIP kernels and the C-ABI host code with hipcc (offload arch
gfx950), then links relative_position_encoding_amd/librelattn.so.  Objects go to
_build/ at the repository root.  Always rebuilds.
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
LIB = os.path.join(PKG, "librelattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["relattn_kernels.hip", "relattn_fwd_bf16.hip", "relattn_window.hip", "relattn_decode.hip",
           "relattn_backward.hip", "relattn_api.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


# Host sanitizers for the C-ABI code (argument checks, plans, the caches): the
# host pass of relattn_api.cpp is built with AddressSanitizer and
# UndefinedBehaviorSanitizer (-Xarch_host: the device code is not
# instrumented), the kernels as usual, into _build/librelattn_san.so.  Run the
# CPU tests against it with
#   RELATTN_LIBRARY=_build/librelattn_san.so ASAN_OPTIONS=detect_leaks=0 \
#   LD_PRELOAD=$(hipcc -print-file-name=libclang_rt.asan-x86_64.so) \
#   python -m pytest tests/test_abi.py -m "not gpu"
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def build_sanitized(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    src = "relattn_api.cpp"
    obj = os.path.join(BUILD, "relattn_api_san.o")
    cmd = [HIPCC] + FLAGS + SAN_FLAGS + ["-O1", "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on the sanitized host build")
    objs = [os.path.join(BUILD, os.path.splitext(x)[0] + ".o") for x in SOURCES if x != src]
    for o in objs:
        if not os.path.exists(o):
            raise RuntimeError(f"{o} missing: run the normal build first")
    out = os.path.join(BUILD, "librelattn_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-fsanitize=address",
           "-fsanitize=undefined", "-shared-libsan", "-o", out] + objs + [obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking librelattn_san.so failed")
    if verbose:
        print(f"built {out}")
    return out


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking librelattn.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized()
    else:
        build()
