"""Loader for the hand-worked examples in tests/golden/worked_examples.json."""

import json
import os
from fractions import Fraction

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def _value(s):
    if s.startswith("2^"):
        return np.float32(2.0 ** int(s[2:]))
    return np.float32(float(s))


def load():
    with open(PATH) as f:
        data = json.load(f)
    out = []
    for c in data["cases"]:
        row = np.array([_value(s) for s in c["row"]], dtype=np.float32)
        draws = [(int(u), int(tok)) for u, tok in c["draws"]]
        ren = [float(Fraction(s)) for s in c["renorm"]]
        out.append((c["name"], row, int(c["top_k"]), float(c["top_p"]), draws, ren))
    return out
