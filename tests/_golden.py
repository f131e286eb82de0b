"""Helpers to read the hand-derived fixtures under tests/golden/."""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hexbytes(s):
    return np.frombuffer(bytes.fromhex(s.replace(" ", "")), dtype=np.uint8).copy()


def num(v):
    if isinstance(v, list):
        v = v[0]
    if isinstance(v, str):
        return {"inf": math.inf, "-inf": -math.inf, "nan": math.nan}[v]
    return float(v)
