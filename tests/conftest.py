import os
import pathlib
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_table(name):
    """Rows of a '|'-separated golden fixture, comments and blanks skipped."""
    rows = []
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        rows.append([c.strip() for c in line.split("|")])
    return rows


def parse_float(tok):
    tok = tok.strip()
    if tok.lower() in ("nan", "inf", "-inf", "+inf"):
        return float(tok)
    if "0x" in tok.lower():
        return float.fromhex(tok)
    return float(tok)


def parse_sparse(tok, conv):
    """'i:v i:v ...' -> dict; '-' -> {}."""
    if tok == "-":
        return {}
    out = {}
    for item in tok.split():
        i, v = item.split(":")
        out[int(i)] = conv(v)
    return out
