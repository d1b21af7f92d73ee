"""Builds q4_K / q5_K raw super-blocks from the hand-worked fixtures under
tests/golden/ (field offsets, code addressing, scale bit packing), independently of
the oracle, for probes whose expected values follow by hand."""
from __future__ import annotations

import numpy as np

from golden_io import kq_code_addressing, kq_layout, kq_scale_bits

LAYOUT = kq_layout()
CODES = kq_code_addressing()
SCALE_BITS = kq_scale_bits()
NAMES = {12: "q4_K", 13: "q5_K"}


def block_info(qtype: int) -> dict:
    return LAYOUT["block"][NAMES[qtype]]


def blank(qtype: int, nblk: int) -> np.ndarray:
    """nblk all-zero super-blocks (d = dmin = 0, every code, scale and min 0)."""
    return np.zeros((nblk, block_info(qtype)["bytes"]), np.uint8)


def set_d(qtype: int, blk: np.ndarray, d: float, dmin: float) -> None:
    info = block_info(qtype)
    blk[info["d"]:info["d"] + 2] = np.array([d], np.float16).view(np.uint8)
    blk[info["dmin"]:info["dmin"] + 2] = np.array([dmin], np.float16).view(np.uint8)


def set_code(qtype: int, blk: np.ndarray, e: int, q: int) -> None:
    """Code of element e (0..255): 4 bits in the code bytes, bit 4 in the fifth bits."""
    info = block_info(qtype)
    row = CODES[e // 32]
    l = e % 32
    i = info["codes"] + row["window"] + l
    if row["nibble"] == "lo":
        blk[i] = (int(blk[i]) & 0xF0) | (q & 15)
    else:
        blk[i] = (int(blk[i]) & 0x0F) | ((q & 15) << 4)
    if info["fifth"] is not None:
        j = info["fifth"] + l
        bit = 1 << row["fifth_bit"]
        blk[j] = (int(blk[j]) | bit) if q & 16 else (int(blk[j]) & ~bit & 0xFF)
    else:
        assert q < 16


def set_scale_min(qtype: int, blk: np.ndarray, s: int, sc: int, m: int) -> None:
    """6-bit scale and min of sub-block s, bit by bit through the packing table."""
    base = block_info(qtype)["scales"]
    for byte, bit, field, sub, dst in SCALE_BITS:
        if sub != s:
            continue
        v = sc if field == "sc" else m
        mask = 1 << bit
        cur = int(blk[base + byte])
        blk[base + byte] = (cur | mask) if (v >> dst) & 1 else (cur & ~mask & 0xFF)
