"""Compile libsdv.so (HIP for gfx950) in-tree with hipcc, and beside it
libsdv_probe.so, the benchmark's plain streaming read (a measurement aid that
is not part of the library's interface)."""

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsdv.so")
SOURCES = ["abi.hip", "schedule.hip", "row_partials.hip", "verify.hip", "markov.hip", "lightspec.hip",
           "uniforms.hip"]
PROBE_LIB = os.path.join(PKG, "libsdv_probe.so")
PROBE_SOURCES = ["probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed FP32 instructions stay disabled: the compiler would otherwise
    # form v_pk_* fp32 ops from plain float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsdv")
    return path


def _compile(sources, out, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-o", tmp] + srcs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
        if err.strip():
            print(err)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Build libsdv.so and libsdv_probe.so next to this file and return the
    library's path (always recompiles)."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
