"""Loader of the hand-worked attention examples in tests/golden/.

Each case gives tiny Q, K, V, dO (leading coordinates only, the rest zero),
the scale, the mask, and O, LSE, dQ, dK, dV worked out by hand, as numbers or
as expressions in ln2, ln3 and ln7 (the derivations are in the file).
"""
import json
import math
import os

import numpy as np

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked_examples.json")
_NAMES = {"ln2": math.log(2.0), "ln3": math.log(3.0), "ln7": math.log(7.0)}


def _value(x):
    if isinstance(x, str):
        return float(eval(x, {"__builtins__": {}}, dict(_NAMES)))
    return float(x)


def _rows(rows, d):
    out = np.zeros((len(rows), d), dtype=np.float64)
    for i, r in enumerate(rows):
        out[i, : len(r)] = [_value(x) for x in r]
    return out


def cases(d):
    """The examples padded to head dimension d, as [S, d] float64 arrays."""
    with open(PATH) as f:
        data = json.load(f)
    out = []
    for c in data["cases"]:
        e = {"name": c["name"], "causal": bool(c["causal"]), "scale": _value(c["scale"])}
        for t in ("q", "k", "v", "do", "o", "dq", "dk", "dv"):
            e[t] = _rows(c[t], d)
        e["lse"] = np.array([_value(x) for x in c["lse"]], dtype=np.float64)
        out.append(e)
    return out
