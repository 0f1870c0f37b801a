"""Readers for the hand-written fixtures under tests/golden/.

Fixture syntax: '#' starts a comment; a comment line of the form
'# key value' directly naming a fixture parameter (scale_code, row_scale) is
read by ``directives``; every other non-blank line is data.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_DIRECTIVES = ("scale_code", "row_scale")


def _raw(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.rstrip("\n") for ln in f]


def lines(name):
    for ln in _raw(name):
        ln = ln.split("#", 1)[0].strip()
        if ln:
            yield ln


def directives(name):
    out = {}
    for ln in _raw(name):
        parts = ln.strip().lstrip("#").split()
        if ln.strip().startswith("#") and len(parts) == 2 and parts[0] in _DIRECTIVES:
            out[parts[0]] = parts[1]
    return out


def code_value_table(name):
    rows = [ln.split()[:2] for ln in lines(name)]
    return np.array([int(c, 16) for c, _ in rows]), np.array([float(v) for _, v in rows])


def value_code_table(name):
    rows = [ln.split()[:2] for ln in lines(name)]
    return np.array([float(v) for v, _ in rows]), np.array([int(c, 16) for _, c in rows])
