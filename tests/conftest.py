import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

# The sanitizer run (tests/test_sanitizers.py) points the suite at instrumented
# builds of the library's host code and of the oracle.
if os.environ.get("MLA_TEST_LIB"):
    from mla_latent_kv_13_amd import build as _libbuild
    _libbuild.LIB_PATH = os.environ["MLA_TEST_LIB"]
if os.environ.get("ORACLE_TEST_LIB"):
    import oracle as _oracle
    _oracle._LIB_PATH = os.environ["ORACLE_TEST_LIB"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()  # builds oracle/_build/liboracle.so with gcc if it is not there yet
    return oracle
