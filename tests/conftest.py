import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Rows of whitespace-separated fields of a golden file, comments stripped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def page_value(name):
    for row in read_golden("page_values.txt"):
        if row[0] == name:
            return float(row[1])
    raise KeyError(name)


def e2m1_table():
    return {int(r[0]): float(r[1]) for r in read_golden("e2m1_values.txt")}
