"""Host-side pieces of bench.py (no GPU): the digest that ties stored HBM
counter readings to the kernel sources, the lookup of those readings, and
the one-GPU contract."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_text_drops_comments_and_blank_lines():
    src = "int a = 1;  // one\n\n/* block\n comment */ int b = 2;\n  // only a comment\nint c;\n"
    assert bench.code_text(src) == "int a = 1;\n int b = 2;\nint c;"


def test_digest_ignores_comments_but_not_code():
    base = {"k.hip": "__global__ void k() { int x = 1; }\n", "a.h": "#define N 4\n"}
    commented = {"k.hip": "// kernel\n__global__ void k() { int x = 1; }  // x\n\n",
                 "a.h": "/* size */\n#define N 4\n"}
    changed = {"k.hip": "__global__ void k() { int x = 2; }\n", "a.h": "#define N 4\n"}
    renamed = {"k2.hip": base["k.hip"], "a.h": base["a.h"]}
    d = bench.kernel_sources_digest(base)
    assert bench.kernel_sources_digest(commented) == d
    assert bench.kernel_sources_digest(changed) != d
    assert bench.kernel_sources_digest(renamed) != d


def test_stored_traffic_needs_matching_sources():
    digest = bench.kernel_sources_digest()
    got = bench.stored_traffic("attn_bwd", "problem5", digest)
    assert got is None or got > 0
    assert bench.stored_traffic("attn_bwd", "problem5", "not-a-digest") is None
    assert bench.stored_traffic("no_such_kernel", "problem5", digest) is None


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
