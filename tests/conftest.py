"""Test configuration: the ``gpu`` marker and import paths.

Tests marked ``gpu`` need an MI355X and the built HIP library; every other test
runs on the CPU (oracle pins, host-side logic, library symbol export).
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")
