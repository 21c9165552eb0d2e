import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


# A sanitized test run (tests/sanitize.py) points the tests at libraries
# built with host-side ASan/UBSan instead of the regular in-tree ones.
if os.environ.get("ATTN_TEST_LIBRARY"):
    import transformer_causal_self_amd as _tca
    _tca.library_path = lambda: os.environ["ATTN_TEST_LIBRARY"]
if os.environ.get("ATTN_TEST_ORACLE"):
    import oracle.build as _ob
    _ob.LIB = os.environ["ATTN_TEST_ORACLE"]
    _ob.SRC_CHECK = False


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
