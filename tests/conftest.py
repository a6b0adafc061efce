import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def by_column_chunks(fn, n, chunk=2048):
    """An oracle result over all n columns, built chunk by chunk to bound host memory:
    fn(columns) returns the rows for that column subset."""
    import numpy as np
    parts = [fn(np.arange(c0, min(c0 + chunk, n))) for c0 in range(0, n, chunk)]
    return np.concatenate(parts, axis=1)


def read_golden(name):
    """Lines of a golden fixture without comments or blanks."""
    path = os.path.join(ROOT, "tests", "golden", name)
    with open(path) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]


def golden_csr_cases():
    cases, cur = [], None
    for parts in read_golden("csr_worked_examples.txt"):
        if parts[0] == "case":
            cur = {"kind": parts[1]}
        elif parts[0] == "end":
            cases.append(cur)
        else:
            cur[parts[0]] = [int(x) for x in parts[1:]]
    return cases
