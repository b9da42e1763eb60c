"""Reader for the text fixtures under tests/golden/.

Format: '#' lines are comments (the citation); ``key: values`` holds one line
of numbers; ``key:`` alone starts a matrix that runs to the next blank line.
"""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    key = None
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        lines = f.read().splitlines() + [""]
    for line in lines:
        s = line.strip()
        if s.startswith("#"):
            continue
        if key is not None:
            if s == "" or (":" in s):
                out[key] = np.array(rows, dtype=np.float64)
                key, rows = None, []
            else:
                rows.append([float(x) for x in s.split()])
                continue
        if not s:
            continue
        k, _, rest = s.partition(":")
        rest = rest.strip()
        if rest == "":
            key = k.strip()
            rows = []
        else:
            vals = [float(x) for x in rest.split()]
            out[k.strip()] = vals[0] if len(vals) == 1 else np.array(vals)
    return out
