import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side oracle runs")
    config.addinivalue_line("markers", "oracle_pool: runs the oracle on every row in worker processes")


def pytest_collection_finish(session):
    """Start the oracle's worker processes before any test touches the GPU,
    when a selected test needs them (see oracle_pool.py)."""
    if any(item.get_closest_marker("oracle_pool") for item in session.items):
        import oracle_pool
        import torch
        if not torch.cuda.is_initialized():
            oracle_pool.start()
