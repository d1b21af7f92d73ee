"""Builders for structured raw q6_K inputs used by the tests.

Element codes are written through the hand-worked addressing table in
tests/golden/q6k_unit_addressing.txt (taken from the unit-load address formulas of
the D4-4 page, §3.2 Excerpt B), never through the oracle or the HIP library, so
a probe built here checks either side's decoder against that table.
"""
from __future__ import annotations

import numpy as np

from golden_io import unit_addressing

_TABLE = unit_addressing()
BLOCK = 210
QH0, SC0, D0 = 128, 192, 208      # field offsets inside a raw block (D4-4 §3.2 Excerpt A)


def blank(N: int, nbe: int, ql: int = 0, qh: int = 0, sc: int = 0, d_bits: int = 0) -> np.ndarray:
    """Raw rows uint8 [N, nbe*210] with every block filled uniformly."""
    blk = np.zeros(BLOCK, np.uint8)
    blk[:QH0] = ql
    blk[QH0:SC0] = qh
    blk[SC0:D0] = np.array([sc], np.int8).view(np.uint8)[0]
    blk[D0] = d_bits & 0xFF
    blk[D0 + 1] = (d_bits >> 8) & 0xFF
    return np.tile(blk, (N, nbe)).reshape(N, nbe * BLOCK).copy()


def set_code(raw: np.ndarray, r: int, b: int, e: int, q: int) -> None:
    """Write 6-bit code q at element e (0..255) of block b of row r."""
    assert 0 <= q < 64 and 0 <= e < 256
    unit = _TABLE[e // 32]
    l = e % 32
    base = b * BLOCK
    i = base + unit["ql_off"] + l
    v = int(raw[r, i])
    if unit["nibble"] == "lo":
        v = (v & 0xF0) | (q & 0x0F)
    else:
        v = (v & 0x0F) | ((q & 0x0F) << 4)
    raw[r, i] = v
    j = base + QH0 + unit["qh_off"] + l
    s = unit["shift"]
    w = int(raw[r, j])
    w = (w & ~(3 << s) & 0xFF) | ((q >> 4) << s)
    raw[r, j] = w


def set_scale(raw: np.ndarray, r: int, b: int, j: int, v: int) -> None:
    raw[r, b * BLOCK + SC0 + j] = np.array([v], np.int8).view(np.uint8)[0]


def set_d(raw: np.ndarray, r: int, b: int, bits: int) -> None:
    raw[r, b * BLOCK + D0] = bits & 0xFF
    raw[r, b * BLOCK + D0 + 1] = (bits >> 8) & 0xFF


def onehot_probe(q0: int, nbe: int = 1, block: int = 0):
    """The one-hot diagonal probe.

    Rows e = 0..255: every element has code 32 (a zero weight) except element e of
    super-block `block`, which has code q0. Sub-block scales sc[j] = j + 1, d = 1.0.
    Returns (raw uint8 [256, nbe*210], qs int8 [256, K], d16 uint16 [256, K/32],
    expected float64 [256 (column), 256 (row)]): column c is one-hot at position
    256*block + c with code 1 and scale 1.0, so the product is diagonal with
    entry (e // 16 + 1) * (q0 - 32).
    """
    K = 256 * nbe
    raw = blank(256, nbe, ql=0x00, qh=0xAA, d_bits=0x3C00)   # code 32 everywhere
    for r in range(256):
        for b in range(nbe):
            for j in range(16):
                set_scale(raw, r, b, j, j + 1)
        set_code(raw, r, block, r, q0)
    qs = np.zeros((256, K), np.int8)
    qs[np.arange(256), 256 * block + np.arange(256)] = 1
    d16 = np.full((256, K // 32), 0x3C00, np.uint16)
    expect = np.diag([(e // 16 + 1) * (q0 - 32) for e in range(256)]).astype(np.float64)
    return raw, qs, d16, expect
