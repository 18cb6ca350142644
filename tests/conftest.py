import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU work (full-size configs)")


def load_fig2():
    """Parse tests/golden/fig2_formats.txt."""
    path = os.path.join(ROOT, "tests", "golden", "fig2_formats.txt")
    spec = {"e": []}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "e":
                spec["e"].append(tuple(int(v) for v in vals))
            elif len(vals) == 1 and key in ("m", "k", "b_row", "b_col"):
                spec[key] = int(vals[0])
            else:
                spec[key] = [int(v) for v in vals]
    return spec


@pytest.fixture(scope="session")
def fig2():
    return load_fig2()


@pytest.fixture(scope="session")
def cfg2():
    import synth
    return synth.config2()
