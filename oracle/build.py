"""Builds the CPU oracle library with the host C compiler.

The oracle is test infrastructure: only the tests, the smoke check and the
benchmark's CPU-baseline leg load it.  It is plain C with no HIP headers.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "bfp8_oracle.c")
LIBRARY = os.path.join(HERE, "libbfp8_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile ``bfp8_oracle.c`` to ``libbfp8_oracle.so`` and return its path.

    No fast-math and no floating-point contraction, so every division,
    product and sum rounds exactly as written in the source.
    """
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           SOURCE, "-o", LIBRARY + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIBRARY + ".tmp", LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
