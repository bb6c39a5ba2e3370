"""Reader for the worked-example fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            vals = [int(v) for v in val.split()]
            out[key.strip()] = vals[0] if len(vals) == 1 else vals
    return out
