import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def _parse_set(tok: str) -> list[int]:
    tok = tok.strip()
    if tok == "-":
        return []
    out = []
    for part in tok.split(","):
        if "-" in part:
            a, b = part.split("-")
            out.extend(range(int(a), int(b) + 1))
        else:
            out.append(int(part))
    return out


def load_partition(F: int):
    """{query frame: (softmax frames, forward frames, backward frames)} from a golden file."""
    table = {}
    with open(os.path.join(GOLDEN, f"partition_F{F}.txt")) as fh:
        for line in fh:
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            qs, s, f, b = [x.strip() for x in line.split("|")]
            for i in _parse_set(qs):
                table[i] = (_parse_set(s), _parse_set(f), _parse_set(b))
    assert sorted(table) == list(range(F))
    return table


@pytest.fixture
def golden_partition():
    return load_partition
