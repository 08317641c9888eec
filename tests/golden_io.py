"""Reader for the text fixtures under tests/golden/.

Format: '#' lines are comments (they carry the citation); a header line
``name rows cols`` is followed by ``rows`` lines of ``cols`` whitespace-separated
entries.  Entries are numbers, or labels when ``labels=True``.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name, labels=False):
    path = os.path.join(GOLDEN, name)
    out = {}
    with open(path, encoding="utf-8") as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
    i = 0
    while i < len(lines):
        key, r, c = lines[i].split()
        r, c = int(r), int(c)
        rows = [lines[i + 1 + j].split() for j in range(r)]
        assert all(len(row) == c for row in rows), f"{name}:{key}: ragged rows"
        out[key] = rows if labels else np.array(rows, dtype=np.float64)
        i += 1 + r
    return out
