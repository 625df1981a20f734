"""Build libtcs.so in-tree with hipcc for gfx950.

    python -m trie_constrained_scoring_amd.build [-v] [--sanitized-host]

Every source is compiled to an object under ``_build/`` (in parallel, warnings as
errors), then linked into ``trie_constrained_scoring_amd/libtcs.so``.  All device
code is compiled with packed-fp32 instruction selection disabled.  --sanitized-host
also builds the host-only sources alone with ASan + UBSan (``_build/``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtcs.so")
ARCH = "gfx950"

SOURCES = ["errors.cpp", "trie_build.cpp", "tcs_api.hip", "k_gemm.hip", "k_lmhead.hip", "k_attn.hip",
           "k_path.hip", "k_letters.hip", "k_decode.hip", "timing.hip"]
# the host-only part (label parsing, trie construction, decision-word cut, status
# messages), also built alone with the address and undefined-behaviour sanitizers
HOST_SOURCES = ["errors.cpp", "trie_build.cpp"]
HOST_SANITIZED_LIB = os.path.join(BUILD, "libtcs_host_sanitized.so")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function",
          "-Werror"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libtcs")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".cpp"):
        cmd = ["g++", *COMMON, "-I/opt/rocm/include", "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, *HIP_FLAGS, "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libtcs.so failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(verbose: bool = False) -> str:
    """The host-only sources alone, with AddressSanitizer and UndefinedBehaviorSanitizer
    (g++; no GPU code), as _build/libtcs_host_sanitized.so.  It exports tcs_trie_build,
    tcs_decision_truncate, tcs_last_error and tcs_version; a process that loads it must
    preload the ASan runtime (g++ -print-file-name=libasan.so)."""
    os.makedirs(BUILD, exist_ok=True)
    tmp = HOST_SANITIZED_LIB + ".tmp"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", f"-I{INCLUDE}", f"-I{CSRC}",
           "-I/opt/rocm/include", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           *[os.path.join(CSRC, f) for f in HOST_SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, HOST_SANITIZED_LIB)
    return HOST_SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--sanitized-host" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
