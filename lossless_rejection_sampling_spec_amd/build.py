"""Build libspecverify.so (HIP, gfx950) in-tree with hipcc.

    python -m lossless_rejection_sampling_spec_amd.build
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", "specverify.hip"), os.path.join(PKG, "csrc", "drain.hip")]
INC = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libspecverify.so")
# Test-only build: every wait between workgroups gives up after one poll, so
# the give-up path (SV_ROW_INTERNAL, the poisoned workspace) runs with every
# kernel exiting normally.  Only the GPU tests load it.
LIB_ONE_POLL = os.path.join(PKG, "libspecverify_onepoll.so")
# The benchmark's streaming-read ceiling kernel (a measurement tool, not the verify).
STREAM_SRC = os.path.join(PKG, "csrc", "stream_read.hip")
LIB_STREAM = os.path.join(PKG, "libsvstream.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every floating-point rounding is the one the source spells out: the
    # element terms recomputed by the final draw match the summed ones bit for bit
    "-ffp-contract=off",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found (set HIPCC)")
    return cand


def _start(out: str, extra: list, verbose: bool, sources=None):
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INC, "-o", out + ".tmp", *(sources or SRC)]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd)


def build(verbose: bool = True) -> str:
    """Compile the library, its one-poll test build and the benchmark's
    streaming-read kernel, side by side (every call)."""
    jobs = [(LIB, _start(LIB, [], verbose)),
            (LIB_ONE_POLL, _start(LIB_ONE_POLL, ["-DSV_SPIN_MAX=1"], verbose)),
            (LIB_STREAM, _start(LIB_STREAM, [], verbose, [STREAM_SRC]))]
    failed = [out for out, proc in jobs if proc.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for out, _ in jobs:
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
