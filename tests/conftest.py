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
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libbigemm.so")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(HERE, "golden")


def pytest_terminal_summary(terminalreporter):
    """Sum of the A/B cells run (tests/harness.py REPORT): one line, and the JSON-lines
    report at $BIGEMM_BI_REPORT when that is set."""
    try:
        import harness
    except ImportError:
        return
    cells = harness.REPORT
    if not cells:
        return
    import collections
    import json
    by = collections.OrderedDict()
    for c in cells:
        n, ab, canon = by.get(c["config"], (0, 0, 0))
        by[c["config"]] = (n + 1, ab + c["ab"], canon + c["canon"])
    parts = ", ".join(f"{k}: {n} cells, {ab} A/B bytes, {canon} vs-alone bytes" for k, (n, ab, canon) in by.items())
    terminalreporter.write_line(f"batch-invariance A/B cells: {len(cells)} in all ({parts})")
    path = os.environ.get("BIGEMM_BI_REPORT")
    if path:
        with open(path, "w") as f:
            for c in cells:
                f.write(json.dumps(c) + "\n")
