"""Build librlk_logprob.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and the
measurement probes of bench.py (librlk_probes.so, include/rlk_probes.h).

    python -m entropy_rlk_logprob_amd.build [--verbose]

Flags that matter for the numerics: -ffp-contract=off (no implicit FMA contraction, so
every rounding is the one the source spells out) and no fast-math.  Packed-fp32 VALU
instruction selection is disabled for the device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "librlk_logprob.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["rlk_api.hip", "rlk_logits.hip", "rlk_linear.hip", "rlk_compare.hip", "rlk_backward.hip",
           "rlk_linear_bwd.hip"]
PROBES_SOURCE = "rlk_probes.hip"
PROBES_PATH = os.path.join(PKG, "librlk_probes.so")
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into the logprob library, then the probe library; returns the
    logprob library's path."""
    _compile([os.path.join(CSRC, s) for s in SOURCES], LIB_PATH, verbose)
    _compile([os.path.join(CSRC, PROBES_SOURCE)], PROBES_PATH, verbose)
    return LIB_PATH


def _compile(srcs: list[str], out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc()] + flags() + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; that warning is noise.
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
