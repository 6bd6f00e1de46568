"""Readers for the small text fixtures under tests/golden/."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line.split()


def max1960_table():
    """{bits: {"centroid": [...], "threshold": [...], "distortion": [...]}}"""
    table = {}
    for fields in _lines("max1960_gaussian_lloyd_max.txt"):
        bits, kind, vals = int(fields[0]), fields[1], [float(v) for v in fields[2:]]
        table.setdefault(bits, {})[kind] = vals
    return table


def pack_example():
    out = {}
    for fields in _lines("pack_d32_b3.txt"):
        if fields[0] == "words":
            out["words"] = [int(v, 16) for v in fields[1:]]
        else:
            out[fields[0]] = int(fields[1])
    return out


def abstract_figures():
    return {f[0]: float(f[1]) for f in _lines("axelram_abstract_figures.txt")}
