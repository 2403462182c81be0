"""Build librtp.so (HIP, gfx950) in place with hipcc.

    python -m head_wise_sparse_rtp_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librtp.so")
SOURCES = ["rtp_api.hip", "rtp_score.hip", "rtp_select.hip", "rtp_attn.hip", "rtp_step.hip",
           "rtp_append.hip", "rtp_prefill.hip", "rtp_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# the benchmark's streaming-read ceiling (not part of librtp)
HBM_READ_SRC = "hbm_read.hip"
HBM_READ_LIB = os.path.join(HERE, "libhbmread.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep fp32 denormals: the indexer fma chain must match IEEE arithmetic
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function",
]


def _compile(srcs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(HERE, "..", "include"), "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in (r.stderr or "").splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError("hipcc failed building %s" % os.path.basename(out))
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, out)
    return out


# the host code (argument checks, size queries, status strings) under AddressSanitizer and
# UndefinedBehaviorSanitizer, for CPU tests that launch no kernel; the device code is built
# plainly (every flag below that names a sanitizer applies to the host pass alone)
SANITIZE_FLAGS = [
    "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Xarch_host", "-g",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
]


def build_host_sanitized(out: str) -> str:
    """Build the host side of librtp.so with ASan and UBSan into `out` (CPU tests only)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ([HIPCC] + SANITIZE_FLAGS + ["-I", os.path.join(HERE, "..", "include"), "-o", tmp] +
           [os.path.join(CSRC, s) for s in SOURCES])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError("hipcc failed building the sanitized host library")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Build librtp.so and the benchmark's libhbmread.so; returns librtp.so's path."""
    _compile([os.path.join(CSRC, s) for s in SOURCES], LIB, verbose)
    _compile([os.path.join(CSRC, HBM_READ_SRC)], HBM_READ_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
