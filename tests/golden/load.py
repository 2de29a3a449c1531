"""Reads the `name = value` fixtures in this folder."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name):
    vals = {}
    with open(os.path.join(HERE, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            vals[k] = float(v) if any(ch in v for ch in ".e") else int(v)
    return vals
