import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: large CPU-side work (full-size oracle runs)")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Parse a golden fixture: `key = value` lines, `#` comments, `---`
    separates cases.  Returns a list of dicts of raw strings."""
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line == "---":
                cases.append(cur)
                cur = {}
                continue
            k, v = line.split("=", 1)
            cur[k.strip()] = v.strip()
    cases.append(cur)
    return cases
