"""Reader for the hand-derived fixtures in tests/golden/*.txt."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    """Returns dict(shape, sampling, mask uint8, sqdist float64)."""
    with open(os.path.join(GOLDEN, name)) as fh:
        lines = [ln.strip() for ln in fh if ln.strip() and not ln.startswith("#")]
    out = {}
    i = 0
    while i < len(lines):
        head = lines[i].split()
        if head[0] == "shape":
            out["shape"] = tuple(int(x) for x in head[1:])
            i += 1
        elif head[0] == "sampling":
            out["sampling"] = tuple(float(x) for x in head[1:])
            i += 1
        elif head[0] in ("mask", "sqdist"):
            n = int(np.prod(out["shape"]))
            vals = []
            i += 1
            while len(vals) < n:
                vals.extend(float(x) for x in lines[i].split())
                i += 1
            arr = np.array(vals).reshape(out["shape"])
            out[head[0]] = arr.astype(np.uint8) if head[0] == "mask" else arr
        else:
            raise ValueError(f"{name}: unexpected line {lines[i]!r}")
    return out


def names():
    return sorted(f for f in os.listdir(GOLDEN) if f.endswith(".txt"))
