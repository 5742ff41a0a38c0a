"""Builds the CPU oracle library with the host C++ compiler.

The oracle is test infrastructure: only the tests, the smoke check and the
benchmark's CPU-baseline leg load it.  It is plain C++17 with no HIP headers.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "bfp8_oracle.cpp")
LIBRARY = os.path.join(HERE, "libbfp8_oracle.so")

# No fast-math and no floating-point contraction, so every division, product
# and sum rounds exactly as written in the source.
CXXFLAGS = ["-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
            "-pthread", "-Wall", "-Wextra"]


def compile_cmd(source: str, output: str, extra=()) -> list:
    """The g++ command line that builds ``source`` into the shared library ``output``."""
    return ["g++"] + CXXFLAGS + list(extra) + [source, "-o", output, "-lm"]


def build(verbose: bool = False) -> str:
    """Compile ``bfp8_oracle.cpp`` to ``libbfp8_oracle.so`` and return its path."""
    cmd = compile_cmd(SOURCE, LIBRARY + ".tmp")
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
