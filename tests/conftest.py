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
    config.addinivalue_line("markers", "slow: full-size workloads (minutes of CPU work)")


# A test may point the binding at another build of the library (the sanitizer
# test's instrumented host code); the product itself always loads its in-tree
# libdattn.so.
if os.environ.get("DATTN_LIBRARY_OVERRIDE"):
    import int8_quantized_kv_amd as _dk

    _dk.library_path = os.environ["DATTN_LIBRARY_OVERRIDE"]
