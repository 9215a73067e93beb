"""Readers for the hand-written text fixtures under tests/golden/."""

from __future__ import annotations

import math
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def e4m3fn_points():
    """[(code, value)] from golden/e4m3fn_spec_points.txt."""
    out = []
    for code, val in _lines("e4m3fn_spec_points.txt"):
        v = math.nan if val == "nan" else float.fromhex(val)
        out.append((int(code, 16), v))
    return out


def fp8_page_fixture():
    """(page bytes, page_size, [(slot, lo, hi, value)]) from golden/fp8_page_ps2.txt."""
    buf = bytearray(1296)
    expects = []
    for parts in _lines("fp8_page_ps2.txt"):
        kind = parts[0]
        if kind == "fill":
            off, cnt, byte = int(parts[1]), int(parts[2]), int(parts[3], 0)
            buf[off: off + cnt] = bytes([byte]) * cnt
        elif kind == "fill16":
            off, cnt, word = int(parts[1]), int(parts[2]), int(parts[3], 0)
            buf[off: off + 2 * cnt] = word.to_bytes(2, "little") * cnt
        elif kind == "expect":
            expects.append((int(parts[1]), int(parts[2]), int(parts[3]), float(parts[4])))
        else:
            raise ValueError(parts)
    return bytes(buf), 2, expects
