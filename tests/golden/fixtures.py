"""Reader for the small text fixtures in this folder (``key = v1 v2 ...``)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            vals = [int(v) for v in val.split()]
            out[key] = vals[0] if len(vals) == 1 else vals
    return out
