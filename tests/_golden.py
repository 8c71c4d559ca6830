"""Readers for the text fixtures under tests/golden/ (each file states its source)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def _float(tok):
    return float.fromhex(tok) if "0x" in tok.lower() else float(tok)


def hand_groups(name="hand_groups.txt"):
    """-> list of dicts {name, x: [float], q: [int], s_bits: int, fill: float}."""
    cases, cur = [], None
    for line in _lines(name):
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = {"name": rest.strip(), "fill": 0.0}
            cases.append(cur)
        elif key == "x":
            cur["x"] = [_float(t) for t in rest.split()]
        elif key == "q":
            cur["q"] = [int(t, 16) for t in rest.split()]
        elif key == "s":
            cur["s_bits"] = int(rest.strip(), 16)
        elif key == "fill":
            cur["fill"] = _float(rest.strip())
    return cases


def table(name):
    """Whitespace-separated numeric rows of a fixture file."""
    return [[_float(t) for t in line.split()] for line in _lines(name)]
