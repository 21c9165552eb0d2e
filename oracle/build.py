"""Build the fp64 CPU oracle (test infrastructure) into oracle/liboracle.so.

The oracle is plain C compiled with gcc and OpenMP.  It is built for the
x86-64-v3 level (AVX2 + FMA) so that the same binary runs on any current x86
host, not only the one it was built on.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
SAN_CC = "/opt/rocm/llvm/bin/clang"   # the sanitizer runtime must match the HIP library's


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB) -> str:
    """Compile oracle.c into `out`.  sanitize=True builds it with clang's
    AddressSanitizer and UndefinedBehaviorSanitizer instead (for the
    sanitized CPU test run, tests/sanitize.py; the process must preload the
    ASan runtime)."""
    if sanitize:
        cmd = [SAN_CC, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    else:
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", out + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
