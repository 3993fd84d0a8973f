"""Build step: compiles the HIP sources in csrc/ into libmoe.so (gfx950), in-tree.

    python -m mixture_experts_ffn_sqrt_amd.build [-v]
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


PEAKS_SRC = os.path.join(HERE, "peaks", "moe_peaks.hip")
PEAKS_LIB = os.path.join(HERE, "libmoe_peaks.so")


def _hipcc(srcs, out, verbose):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
           # packed fp32 instructions stay off (plain scalar fp32 code only)
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-o", out + ".tmp"] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def build_peaks(verbose: bool = False) -> str:
    """The chip-ceiling microbenchmarks (include/moe_peaks.h): libmoe_peaks.so."""
    return _hipcc([PEAKS_SRC], PEAKS_LIB, verbose)


def build(verbose: bool = False) -> str:
    _hipcc(sources(), LIB, verbose)
    build_peaks(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
