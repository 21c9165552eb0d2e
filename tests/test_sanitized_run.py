"""Under tests/sanitize.py: the libraries this process runs are the
sanitized builds and the ASan runtime is loaded (else the run proves
nothing).  Skipped in ordinary runs."""
import os

import pytest

import oracle
import transformer_causal_self_amd as tca

pytestmark = pytest.mark.skipif(not os.environ.get("ATTN_TEST_LIBRARY"),
                                reason="only in the sanitized CPU run")


def test_sanitized_libraries_are_the_ones_loaded():
    tca.load_library()
    oracle.num_threads()
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert os.environ["ATTN_TEST_LIBRARY"] in maps
    assert os.environ["ATTN_TEST_ORACLE"] in maps
    assert "libclang_rt.asan" in maps
    assert "libattn_mi355.so" not in maps.replace(os.environ["ATTN_TEST_LIBRARY"], "")


def test_sanitizer_symbols_in_the_builds():
    import subprocess
    for lib in (os.environ["ATTN_TEST_LIBRARY"], os.environ["ATTN_TEST_ORACLE"]):
        syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, lib
