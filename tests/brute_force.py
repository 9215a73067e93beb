"""Brute-force sparse MLA decode for tiny inputs: a second, independent reading.

Pure-Python loops with math.fsum over the selected rows; number formats are decoded
with torch's own float8_e4m3fn and bfloat16 types (library routines), and the cache
offsets are worked out here from the layout definition, not taken from the oracle.
Used only to pin the oracle on inputs of a few entries and heads.
"""

from __future__ import annotations

import math

import torch


def _bf16_list(raw: bytes):
    t = torch.frombuffer(bytearray(raw), dtype=torch.bfloat16)
    return [float(x) for x in t.double().tolist()]


def _e4m3_list(raw: bytes):
    t = torch.frombuffer(bytearray(raw), dtype=torch.uint8).view(torch.float8_e4m3fn)
    return [float(x) for x in t.double().tolist()]


def entry(cache: bytes, fmt: str, page_size: int, slot: int, kv_scale: float = 1.0):
    """Dequantized 576-vector of one cache slot."""
    page, row = divmod(slot, page_size)
    if fmt == "bf16":
        base = page * 1152 * page_size + row * 1152
        return _bf16_list(cache[base: base + 1152])
    if fmt == "fp8t":
        base = page * 576 * page_size + row * 576
        return [v * kv_scale for v in _e4m3_list(cache[base: base + 576])]
    base = page * 648 * page_size
    lat = _e4m3_list(cache[base + 512 * row: base + 512 * row + 512])
    rope_at = base + 512 * page_size + 128 * row
    rope = _bf16_list(cache[rope_at: rope_at + 128])
    sc_at = base + 640 * page_size + 8 * row
    sc = cache[sc_at: sc_at + 8]
    return [lat[d] * math.ldexp(1.0, sc[d // 64] - 127) for d in range(512)] + rope


def decode_row(q_row, cache: bytes, fmt: str, page_size: int, idx_row, slot_of, scale, sinks,
               kv_scale: float = 1.0):
    """q_row: list of H lists of 576 floats; idx_row: list of ints; slot_of(t) -> slot.

    Returns (o, lse): H lists of 512 floats and H floats.  Each list position with an
    index other than -1 is one term (a repeated index counts as often as it appears).
    """
    ks = [entry(cache, fmt, page_size, slot_of(t), kv_scale) for t in idx_row if t != -1]
    outs, lses = [], []
    for h, qh in enumerate(q_row):
        sig = -math.inf if sinks is None else float(sinks[h])
        s = [scale * math.fsum(qh[d] * k[d] for d in range(576)) for k in ks]
        if not s:
            outs.append([0.0] * 512)
            lses.append(sig)
            continue
        m = max(s + [sig])
        w = [math.exp(x - m) for x in s]
        ws = 0.0 if sig == -math.inf else math.exp(sig - m)
        z = math.fsum(w + [ws])
        outs.append([math.fsum(w[j] * ks[j][d] for j in range(len(ks))) / z for d in range(512)])
        lses.append(m + math.log(z))
    return outs, lses
