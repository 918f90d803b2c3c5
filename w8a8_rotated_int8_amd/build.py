"""Build libconvrot.so (every HIP kernel of the package) for gfx950 with hipcc.

The library is built in-tree, next to this file.  Flags:
  -O3 --offload-arch=gfx950            CDNA4 only
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE fp32 division (per-row scales)
  -Xclang -target-feature -Xclang -packed-fp32-ops   (minus sign: disabled) no
                                       packed fp32 instructions are generated
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libconvrot.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


PROBE_SRC = os.path.join(HERE, "probe", "hbm_stream.hip")
PROBE_LIB = os.path.join(HERE, "libhbm_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The streaming reference bench.py times beside the HBM-bound kernels."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(HERE, "..", "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
