"""Small text fixtures holding what the pages print for their worked examples, each file headed by
the passage it comes from, and a reader for them.

Format: '#' starts a comment line; every other line is 'key: value'.  A value made of
'name=value' tokens is returned as a dict of strings; a plain value as a string.  A key may repeat:
its values are kept in file order."""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _value(text: str):
    toks = text.split()
    if toks and all("=" in t for t in toks):
        return dict(t.split("=", 1) for t in toks)
    if len(toks) > 1 and "=" in toks[1]:
        head, rest = toks[0], toks[1:]
        out = dict(t.split("=", 1) for t in rest)
        out[""] = head
        return out
    return text.strip()


def load(name: str) -> dict:
    """Reads tests/golden/<name>; returns {key: [values in file order]}."""
    out: dict = {}
    with open(os.path.join(HERE, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out.setdefault(key.strip(), []).append(_value(val))
    return out


def one(fix: dict, key: str):
    (v,) = fix[key]
    return v


def ints(text: str) -> list:
    return [int(x) for x in text.split(",")]


def flag(text: str) -> bool:
    assert text in ("True", "False"), text
    return text == "True"
