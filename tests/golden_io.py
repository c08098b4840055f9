"""Reader for the hand-worked fixtures under tests/golden/ ('|'-separated fields, ';' separates rows)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _field(s):
    rows = [r.split() for r in s.split(";")]
    return rows


def read_cases(name):
    cases = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            cases.append([_field(p) for p in line.split("|")])
    return cases


def arr(field, dtype=np.float64):
    return np.array([[float(v) for v in row] for row in field], dtype=dtype)


def scalar(field):
    return float(field[0][0])
