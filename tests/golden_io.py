"""Reader for the hand-worked fixtures under tests/golden/ (simple 'key values...' blocks)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_cases(name):
    cases, cur = {}, None
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
            elif key == "end":
                cases[cur["name"]] = cur
                cur = None
            elif cur is not None:
                cur[key] = vals
    return cases


def read_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()[:2]
                out[k] = int(v)
    return out
