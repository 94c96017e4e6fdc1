"""Reader for the cited text fixtures under tests/golden/."""
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def records(name):
    """Non-comment lines of a fixture, split on whitespace."""
    out = []
    with open(os.path.join(HERE, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def first(name, key):
    for rec in records(name):
        if rec[0] == key:
            return rec[1:]
    raise KeyError(key)


def all_of(name, key):
    return [rec[1:] for rec in records(name) if rec[0] == key]
