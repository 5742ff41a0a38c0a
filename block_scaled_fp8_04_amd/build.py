"""Builds libbfp8.so (the HIP library behind include/bfp8.h) for gfx950 with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libbfp8.so")
SOURCES = ["api.hip", "quant.hip", "dequant.hip", "gemm.hip", "grouped.hip", "gemm_bf16.hip", "moe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -O3, no fast-math: fp32 division stays correctly rounded (act_quant relies on
# it).  Packed fp32 instructions are disabled for the device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-rdc", "-Wall", "-Wno-unused-result"]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source into ``libbfp8.so``; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [HIPCC] + FLAGS + list(extra_flags or []) + ["-I", os.path.join(ROOT, "include")] + \
        srcs + ["-o", LIBRARY + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only packed-fp32 feature and says so; drop that line
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
