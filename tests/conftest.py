import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden_path(name):
    return os.path.join(GOLDEN, name)


def read_golden_floats(name):
    vals = []
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float(line))
    return vals


def read_golden_figures(name):
    out = {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                key, val = line.split()[:2]
                out[key] = float(val)
    return out
