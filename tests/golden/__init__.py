"""Worked examples printed on the pages, stored as small text fixtures.

Each file starts with comment lines naming the page and section it comes from;
the remaining lines are ``name = numbers``.  No value here comes from the GPU
library.
"""
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(_HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = np.array([float(x) for x in val.split()], dtype=np.float64)
    return out
