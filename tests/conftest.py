import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host time for the oracle)")


def load_golden(name):
    """Parse a tests/golden/*.txt worked example: `key = expression` lines, where expressions
    are Python literals/arithmetic over sqrt, sin, cos, exp, log, pi."""
    import math

    env = {"sqrt": math.sqrt, "sin": math.sin, "cos": math.cos, "exp": math.exp,
           "log": math.log, "pi": math.pi, "__builtins__": {}}
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, expr = line.split("=", 1)
            out[key.strip()] = eval(expr.strip(), env)  # fixture text is ours, math-only namespace
    return out


@pytest.fixture
def golden():
    return load_golden
