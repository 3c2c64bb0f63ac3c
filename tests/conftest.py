import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_sessionstart(session):
    """In the sanitizer child run (tests/test_sanitizers.py), load the
    sanitizer builds of the oracle and of the host side of the library in
    place of the regular ones."""
    so = os.environ.get("QMV_SANITIZED_ORACLE")
    if so:
        import oracle
        oracle.use_library(oracle.load_library(so))
    sl = os.environ.get("QMV_SANITIZED_LIB")
    if sl:
        from block_quantized_matvec_gguf_amd import binding
        binding.load(sl)


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a golden fixture: 'key: value' lines, '#' comments; repeated keys
    collect into a list."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out.setdefault(key.strip(), []).append(val.strip())
    return out


@pytest.fixture(scope="session")
def golden():
    return read_golden
