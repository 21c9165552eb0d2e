"""Run the CPU test suite against host code built with AddressSanitizer and
UndefinedBehaviorSanitizer: the library's host side (plan, validation, entry
points, launchers; device code is unchanged) and the fp64 oracle.

    python tests/sanitize.py [extra pytest args]

Both libraries are built with ROCm's clang into _build_san/ folders, the ASan
runtime is preloaded into the test process (Python itself is not
instrumented), leak checking is off (the interpreter's own allocations are
not ours to free), and any report or undefined-behaviour finding ends the run
with an error.  No GPU is needed or used.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import build as oracle_build                          # noqa: E402
from transformer_causal_self_amd import build as hip_build        # noqa: E402

PKG_SAN = os.path.join(ROOT, "transformer_causal_self_amd", "_build_san")
ORACLE_SAN = os.path.join(ROOT, "oracle", "_build_san")


def asan_runtime() -> str:
    r = subprocess.run([oracle_build.SAN_CC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return r.stdout.strip()


def main(argv):
    os.makedirs(PKG_SAN, exist_ok=True)
    os.makedirs(ORACLE_SAN, exist_ok=True)
    lib = hip_build.build(sanitize=True, out=os.path.join(PKG_SAN, "libattn_mi355.so"))
    olib = oracle_build.build(sanitize=True, out=os.path.join(ORACLE_SAN, "liboracle.so"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["ATTN_TEST_LIBRARY"] = lib
    env["ATTN_TEST_ORACLE"] = olib
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu",
           "-p", "no:cacheprovider"] + argv
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
