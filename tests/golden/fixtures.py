"""Reader for the small text fixtures in this folder (worked examples from the pages)."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    """Parse ``key: value`` lines and the ``input:`` block of a fixture file."""
    out: dict = {}
    rows = []
    reading_input = False
    with open(os.path.join(HERE, name)) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            if reading_input and ":" not in line:
                rows.append([int(v) for v in line.split()])
                continue
            reading_input = False
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "input":
                reading_input = True
                continue
            out[key] = val
    out["input"] = np.array(rows, dtype=np.uint32)
    return out
