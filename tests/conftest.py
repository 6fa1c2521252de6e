"""Shared pytest setup: the `gpu` marker and import paths.

Tests marked `gpu` need a ROCm device and the built HIP library; everything else
runs on a CPU-only machine."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built libqlin")
