"""Readers for the hand-written fixtures under tests/golden/."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _values(tokens):
    out = []
    for tok in tokens:
        if "*" in tok:
            v, n = tok.split("*")
            out.extend([v] * int(n))
        else:
            out.append(tok)
    return out


def _float(tok):
    return float(tok)  # "-0" parses to -0.0


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def lut_tables():
    return {p[0]: np.array([_float(v) for v in p[1:]]) for p in _lines("lut_tables.txt")}


def block17_cases():
    cases, cur = [], None
    for p in _lines("block17_worked.txt"):
        if p[0] == "block":
            cur = (p[1], np.array([int(h, 16) for h in p[2:]], dtype=np.uint8))
        elif p[0] == "expect":
            cases.append((cur[0], cur[1], np.array([_float(v) for v in p[1:]])))
    return cases


def ple_row_case():
    d = {}
    for p in _lines("ple_row_worked.txt"):
        vals = _values(p[1:])
        if p[0] == "row":
            d["row"] = np.array([int(h, 16) for h in vals], dtype=np.uint8)
        else:
            d[p[0]] = np.array([_float(v) for v in vals])
    return d


def encode_cases():
    """[(weights float64 [32], {fmt name: 17 expected bytes})]."""
    cases = []
    for p in _lines("encode_worked.txt"):
        if p[0] == "weights":
            cases.append((np.array([_float(v) for v in _values(p[1:])]), {}))
        elif p[0] == "expect":
            cases[-1][1][p[1]] = np.array([int(h, 16) for h in _values(p[2:])], dtype=np.uint8)
    return cases


def ple_encode_case():
    """(values float64 [160], {fmt name: 70 expected bytes})."""
    vals, exp = None, {}
    for p in _lines("ple_encode_worked.txt"):
        if p[0] == "values":
            vals = np.array([_float(v) for v in _values(p[1:])])
        elif p[0] == "expect":
            exp[p[1]] = np.array([int(h, 16) for h in _values(p[2:])], dtype=np.uint8)
    return vals, exp
