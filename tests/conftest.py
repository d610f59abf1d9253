"""Shared test configuration.

Tests marked ``gpu`` need an MI355X and the built HIP library; everything else
runs on the CPU.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU and the built libw4a4.so")


@pytest.fixture(scope="session")
def golden():
    import json
    with open(os.path.join(ROOT, "tests", "golden", "rotate_notes_examples.json")) as f:
        return json.load(f)


@pytest.fixture
def hooks(monkeypatch):
    """Route the binding to the test build of the library (libw4a4_test.so), whose kernel choice
    reads the W4A4_* path-forcing variables; returns ``monkeypatch`` for setting them."""
    from w4a4_bit_quantized_amd import binding
    monkeypatch.setattr(binding, "_LIB", _test_lib())
    return monkeypatch


_TEST_LIB = []


def _test_lib():
    from w4a4_bit_quantized_amd import binding
    if not _TEST_LIB:
        _TEST_LIB.append(binding.open_library(binding.test_library_path()))
    return _TEST_LIB[0]
