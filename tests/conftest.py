"""Test configuration: marker registration and import path.

`-m "not gpu"` runs the oracle pins, host-side logic and the C-ABI load/validation checks;
`-m gpu` runs the parity tests that call the HIP library through its C ABI.
"""
import os
import sys

import torch  # noqa: F401  (load torch's HIP runtime before any native library of ours)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
