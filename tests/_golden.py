"""Reader for the key = value fixtures under tests/golden/."""
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (x.strip() for x in line.split("=", 1))
            out[k] = float(v) if "." in v else int(v)
    return out
