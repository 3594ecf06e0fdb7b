import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case, minutes of work")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_path(name: str) -> str:
    return os.path.join(GOLDEN, name)


def golden_rows(name: str):
    """Non-comment lines of a golden fixture, split on '|'."""
    out = []
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            out.append([part.strip() for part in line.split("|")])
    return out


def golden_kv(name: str):
    """key: value lines of a golden fixture."""
    out = {}
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def parse_matrix(text: str):
    import numpy as np
    return np.array([[float(x) for x in row.split()] for row in text.split(";")])
