"""Build libattn_mi355.so (host plan + gfx950 HIP kernels) in-tree.

    python -m transformer_causal_self_amd.build [-v]

Every source is compiled with hipcc for gfx950 only, packed-FP32 instruction
selection disabled, into transformer_causal_self_amd/_build/, then linked
into transformer_causal_self_amd/libattn_mi355.so.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn_mi355.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["plan.cpp", "rope_qkv.hip", "attn_fwd.hip", "attn_bwd.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (the sanitized CPU
# test run, tests/sanitize.py): every flag applies to the host pass only.
SAN_FLAGS = []
for _f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g"):
    SAN_FLAGS += ["-Xarch_host", _f]


def _compile(src: str, verbose: bool, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, flush=True)
    return obj


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB) -> str:
    """Compile and link the library into `out`.  sanitize=True adds host-side
    ASan/UBSan (device code unchanged) and uses its own object directory."""
    build_dir = BUILD + ("_san" if sanitize else "")
    os.makedirs(build_dir, exist_ok=True)
    extra = SAN_FLAGS if sanitize else []
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
