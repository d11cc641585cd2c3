import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


# Test-only library overrides (the CPU sanitizer run in tests/sanitize/ points
# them at instrumented builds of the host layer and of the C oracle).
if os.environ.get("UA_TEST_LIBRARY"):
    from paged_varlen_flashattention_amd import _binding as _b
    _b.LIB_PATH = os.environ["UA_TEST_LIBRARY"]
if os.environ.get("UA_TEST_ORACLE_LIBRARY"):
    import oracle as _o
    _o.LIB = os.environ["UA_TEST_ORACLE_LIBRARY"]
