"""Compiles libqrow.so (the HIP kernels and the C-ABI) for gfx950 in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "qrow.hip"),
           os.path.join(HERE, "csrc", "imatrix.hip"),
           os.path.join(HERE, "csrc", "matmul.hip"),
           os.path.join(HERE, "csrc", "stats.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqrow.so")
# measurement only: VALU issue rates of the instruction classes the kernels
# use (loaded by bench.py; not part of the quantization path or its C-ABI)
PROBE_SOURCES = [os.path.join(HERE, "csrc", "valu_rates.hip")]
PROBE_LIB = os.path.join(HERE, "libqrow_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every float operation as written: no contraction, no fast-math,
    # correctly rounded fp32 division and square root
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(sources, lib, verbose):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-o", tmp, *sources]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    _hipcc(PROBE_SOURCES, PROBE_LIB, verbose)
    return _hipcc(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
