"""Readers for the hand-derived fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_records(name):
    """Map each record key to a list of int lists (one per line with that key)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "kv_row":
                row = [tuple(int(x) for x in v.split(":")) for v in vals]
            else:
                row = [int(x) for x in vals]
            out.setdefault(key, []).append(row)
    return out


def runs_to_positions(runs):
    pos = []
    for a, b in zip(runs[0::2], runs[1::2]):
        pos.extend(range(a, b))
    return pos
