"""Build libdsa.so (all HIP kernels + the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed fp32 arithmetic on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-Wno-pass-failed",
]


PROBE_SRC = os.path.join(PKG, "probe", "read_stream.hip")
PROBE_LIB = os.path.join(PKG, "libdsa_probe.so")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Build libdsa.so (the library) and libdsa_probe.so (the read-stream
    reference kernel that the benchmark quotes the score kernel against)."""
    _hipcc(sources(), LIB, verbose)
    _hipcc([PROBE_SRC], PROBE_LIB, verbose)
    return LIB


def _hipcc(srcs: list[str], lib: str, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in r.stderr.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
