"""Reader for the `key = value` golden fixtures in this folder."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (t.strip() for t in line.split("=", 1))
            out[k] = float(v) if any(ch in v for ch in ".e") else int(v)
    return out
