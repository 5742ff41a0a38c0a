"""Builds libbfp8.so (the HIP library behind include/bfp8.h) for gfx950 with hipcc.

Each source is compiled to its own object (in parallel, in a temporary folder),
then the objects are linked into the shared library.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "libbfp8.so")
SOURCES = ["api.hip", "quant.hip", "dequant.hip", "gemm.hip", "grouped.hip", "gemm_bf16.hip",
           "moe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -O3, no fast-math: fp32 division stays correctly rounded (act_quant relies on
# it).  Packed fp32 instructions are disabled for the device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-fno-gpu-rdc", "-Wall", "-Wno-unused-result"]
# extra hipcc flags for single sources (none at present)
PER_FILE = {}
# hipcc's host pass does not know the device-only packed-fp32 feature and says so
NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    return res.returncode, err


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every HIP source and link ``libbfp8.so``; returns its path."""
    with tempfile.TemporaryDirectory(prefix="bfp8_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            cmd = [HIPCC] + FLAGS + PER_FILE.get(src, []) + list(extra_flags or []) + \
                ["-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
            return (src,) + _run(cmd, verbose)
        with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
            results = list(ex.map(compile_one, SOURCES))
        for src, rc, err in results:
            if rc != 0:
                sys.stderr.write(err + "\n")
                raise RuntimeError(f"hipcc failed on {src} with status {rc}")
            if verbose and err.strip():
                sys.stderr.write(err + "\n")
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        rc, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs +
                       ["-o", LIBRARY + ".tmp"], verbose)
        if rc != 0:
            sys.stderr.write(err + "\n")
            raise RuntimeError(f"linking libbfp8.so failed with status {rc}")
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
