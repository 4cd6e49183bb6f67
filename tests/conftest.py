import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


# A test of the library under a host sanitizer points the binding at that
# build of it (tests/test_host_asan.py); nothing else sets this.
if os.environ.get("RKV_TEST_LIB"):
    from decode_kv_cache_03_amd import _lib as _rkv_lib
    _rkv_lib.LIB_PATH = os.environ["RKV_TEST_LIB"]
