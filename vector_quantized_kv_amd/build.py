"""Build libcommvq.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcommvq.so")
SOURCES = ["api.cpp", "kernels.hip", "attn.hip", "attn_f16.hip", "attn_wide.hip", "noalloc.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# measurement probes for the benchmark (HBM read stream, LDS random gathers): a library of their own
PROBES_LIB = os.path.join(PKG, "libcommvq_probes.so")
PROBES_SOURCES = ["probes.hip"]


def _hipcc(sources, out: str, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp] + [os.path.join(CSRC, s) for s in sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if proc.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Builds libcommvq.so (the C ABI and every kernel of the path) and libcommvq_probes.so (measurement
    probes used by the benchmark); returns the path of libcommvq.so."""
    _hipcc(PROBES_SOURCES, PROBES_LIB, verbose)
    return _hipcc(SOURCES, LIB, verbose)


HOST_CHECK_LIB = os.path.join(ROOT, "_build", "libcommvq_hostcheck.so")
HOST_CHECK_SOURCES = ["api.cpp", "host_stubs.cpp"]
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined"]


def build_host_check() -> str:
    """Host-only build of the C ABI (argument checks, sizing, error reporting) with AddressSanitizer and
    UndefinedBehaviorSanitizer, compiled by g++ with every device launch replaced by a stub that reports
    hipErrorNoDevice (csrc/host_stubs.cpp). Load it with COMMVQ_LIBRARY and the sanitizer runtimes preloaded."""
    os.makedirs(os.path.dirname(HOST_CHECK_LIB), exist_ok=True)
    tmp = HOST_CHECK_LIB + ".tmp"
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared", *SANITIZE_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I",
           "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC, "-o", tmp] + \
          [os.path.join(CSRC, s) for s in HOST_CHECK_SOURCES]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("g++ failed building the host-check library")
    os.replace(tmp, HOST_CHECK_LIB)
    return HOST_CHECK_LIB


if __name__ == "__main__":
    print(build(verbose=True))
