"""Shared pytest configuration.

Markers:
  gpu -- needs an MI355X (gfx950) GPU and the built libtgs.so; run with
         `pytest -m gpu`.  Everything else runs on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built libtgs.so")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    oracle.build()
    return oracle


@pytest.fixture(scope="session")
def tgs_gpu():
    """The binding, with a GPU present (fails loudly otherwise: a gpu test must
    never pass without running the HIP path)."""
    import torch
    assert torch.cuda.is_available(), "gpu test run without a visible GPU"
    import top_gradient_sparsification_amd as tgs
    tgs.library()
    return tgs
