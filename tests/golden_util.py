"""Reader of the hand-derived fixtures under tests/golden/."""
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def num(tok: str):
    t = tok.lower()
    if t.startswith(("0x", "-0x")):
        return int(t, 16)
    return float(tok)


def rows(name: str):
    """Data lines of a fixture as lists of tokens (comments dropped)."""
    out = []
    with open(os.path.join(HERE, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out
