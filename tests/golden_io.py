"""Readers for the hand-derived fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    """Whitespace-separated data rows of a fixture, comments dropped."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def fields(name):
    """`key = v1 v2 ...` lines of a fixture as a dict of token lists."""
    out = {}
    for r in rows(name):
        if len(r) >= 2 and r[1] == "=":
            out[r[0]] = r[2:]
    return out
