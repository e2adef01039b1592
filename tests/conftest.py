import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def golden_path(name: str) -> str:
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden_examples(name: str):
    """Parse 'key: values' blocks separated by blank lines."""
    blocks, cur = [], {}
    for line in open(golden_path(name)):
        line = line.rstrip("\n")
        if line.startswith("#"):
            continue
        if not line.strip():
            if cur:
                blocks.append(cur)
                cur = {}
            continue
        k, v = line.split(":", 1)
        cur[k.strip()] = v.strip()
    if cur:
        blocks.append(cur)
    return blocks
