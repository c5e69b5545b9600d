"""Build the gfx950 shared library ``libspecverify.so`` in-tree with hipcc.

Usage: ``python -m rejection_sampling_verify_scaled_amd.build`` (or call
``build()``).  Every build compiles from source; nothing is cached elsewhere.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", name)
        for name in ("spec_verify.hip", "early_exit.hip", "draft_sample.hip", "commit_tokens.hip",
                     "tree_verify.hip")]
SRC = SRCS[0]  # the verify kernel's source (its sha256 keys the committed traffic counters)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
# The same sources with every bounded wait cut to a single load: a test build
# in which waits expire, to check that the kernels then still exit and fail
# only the requests they could not finish (never loaded by the product path).
LIB_SPIN0 = os.path.join(PKG, "libspecverify_spin0.so")
SPIN0_FLAGS = ("-DSV_SPIN_LIMIT=0u",)
# The same sources with the verify kernel's stage timestamps compiled in
# (SV_TRACE): a measurement build for `bench.py --stage-trace`.
LIB_TRACE = os.path.join(PKG, "libspecverify_trace.so")
TRACE_FLAGS = ("-DSV_TRACE",)
# Issue rates of the VALU instruction classes the samplers use: a measurement
# library of its own for `bench.py --valu-rates` (not part of the verify path).
LIB_RATES = os.path.join(PKG, "libspecverify_rates.so")
RATES_SRC = os.path.join(PKG, "csrc", "valu_rates.hip")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # no implicit multiply-add fusion: the kernel relies on fl(m*c) being the
    # same rounded product everywhere it appears; every intended fma is explicit
    "-ffp-contract=off",
    # packed-FP32 instructions stay off: hipcc would otherwise form them itself
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIB, extra=(), verbose: bool = False, srcs=None) -> str:
    """Compile the HIP sources to ``out`` (a fresh temp file renamed into place)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, f"-I{INCLUDE}", "-o", tmp, *(srcs or SRCS)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> None:
    """The product library, the expired-wait test build, the stage-trace build
    and the VALU issue-rate library."""
    build(verbose=verbose)
    build(out=LIB_SPIN0, extra=SPIN0_FLAGS, verbose=verbose)
    build(out=LIB_TRACE, extra=TRACE_FLAGS, verbose=verbose)
    build(out=LIB_RATES, verbose=verbose, srcs=[RATES_SRC])


if __name__ == "__main__":
    if sys.argv[1:] == ["--all"]:
        build_all(verbose=True)
        print(LIB, LIB_SPIN0, LIB_TRACE, LIB_RATES)
    else:
        build(verbose=True, extra=sys.argv[1:])
        print(LIB)
