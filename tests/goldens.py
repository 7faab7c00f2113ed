"""Readers for the hand-worked fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name):
    """Parse a fixture: '#' comments; each other line is 'key value...'.
    Repeated keys accumulate into lists."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out.setdefault(key, []).append(vals)
    return out


def ints(vals):
    return [int(v) for v in vals]


def hex16(vals):
    return np.array([int(v, 16) for v in vals], dtype=np.uint16)
