"""Reader for the hand-worked text fixtures under tests/golden/ ("key: values" lines,
'#' comments, ';' separating matrix rows)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.strip()
    return out


def vec(s, dtype=np.float64):
    s = s.strip()
    if not s:
        return np.zeros(0, dtype)
    return np.array([float(t) for t in s.split()], dtype)


def mat(s, dtype=np.float64):
    return np.array([[float(t) for t in row.split()] for row in s.split(";")], dtype)


def ints(s):
    s = s.strip()
    return [int(t) for t in s.split()] if s else []
