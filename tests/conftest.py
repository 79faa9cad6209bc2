"""Test configuration: the repository root on sys.path and the `gpu` marker.

Tests marked `gpu` need an MI355X (gfx950) and the built HIP libraries; all
other tests run on the CPU."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP libraries")
