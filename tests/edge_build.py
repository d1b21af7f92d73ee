"""Raw q6_K / q4_K / q5_K rows and q8 planes at the edges of their operand ranges.

The generators of the workloads keep d > 0 and the q6_K sub-block scales in
[-32, 31] (D4-4 §3.3 asks that scales be synthesized deliberately rather than as
random fp16 bits). These builders place the remaining legal values by hand, field
by field at the block offsets of the raw super-block (q6_K: D4-4 §3.2 Excerpt A;
q4_K / q5_K: the public GGUF definitions), so that a GEMV is exercised on:
  - negative, subnormal, largest finite and negative-zero fp16 scales d (and dmin);
  - int8 sub-block scales -128, -1, 0 and 127 (q6_K), 6-bit scales and mins 0 and
    63 (q4_K / q5_K);
  - codes 0 and 63 (q6_K), 0 and 15 / 31 (q4_K / q5_K);
  - q8 activations -128 and 127 with block scales of either sign, subnormal,
    largest finite and zero.
Every fp16 value written is finite: random fp16 bit patterns would include NaN,
whose comparisons make equal results look different (D4-4 §3.3).
"""
from __future__ import annotations

import numpy as np

Q4_K, Q5_K, Q6_K = 12, 13, 14
BLOCK = {Q4_K: 144, Q5_K: 176, Q6_K: 210}

F16_ONE, F16_MINUS_ONE = 0x3C00, 0xBC00
F16_MAX, F16_MINUS_MAX = 0x7BFF, 0xFBFF
F16_MINUS_ZERO = 0x8000
F16_SUBNORMALS = (0x0001, 0x03FF, 0x0200, 0x8001, 0x83FF)


def _bytes(rng, n):
    return rng.integers(0, 256, size=n, dtype=np.uint8)


def _f16_random_normal(rng, n, signed=True):
    """fp16 bit patterns of normal numbers, exponent uniform over the whole range."""
    e = rng.integers(1, 31, size=n)                  # biased exponent 1..30
    m = rng.integers(0, 1024, size=n)
    s = rng.integers(0, 2, size=n) if signed else np.zeros(n, np.int64)
    return ((s << 15) | (e << 10) | m).astype(np.uint16)


def _put16(blk, bits):
    """fp16 bits (scalar or per block) into the 2 bytes at blk[..., 0:2]."""
    bits = np.asarray(bits, np.uint16)
    blk[..., 0] = (bits & 0xFF).astype(np.uint8)
    blk[..., 1] = (bits >> 8).astype(np.uint8)


Q6K_KINDS = ("min_codes_min_scale", "max_codes_max_scale_neg_d", "extreme_scales_neg_d",
             "subnormal_d", "max_d", "neg_zero_d", "full_range")


def q6k_blocks(kind: str, n: int, rng) -> np.ndarray:
    """n raw q6_K blocks [n, 210] of one kind."""
    blk = np.zeros((n, 210), np.uint8)
    if kind == "min_codes_min_scale":        # every code 0, every scale -128, d = 1
        blk[:, 192:208] = 0x80
        _put16(blk[:, 208:210], F16_ONE)
    elif kind == "max_codes_max_scale_neg_d":  # every code 63, every scale 127, d = -1
        blk[:, 0:192] = 0xFF
        blk[:, 192:208] = 127
        _put16(blk[:, 208:210], F16_MINUS_ONE)
    elif kind == "extreme_scales_neg_d":     # scales -128, -1, 0, 127; d < 0
        blk[:, 0:192] = _bytes(rng, n * 192).reshape(n, 192)
        blk[:, 192:208] = rng.choice(np.array([0x80, 0xFF, 0x00, 0x7F], np.uint8), size=(n, 16))
        _put16(blk[:, 208:210], _f16_random_normal(rng, n) | 0x8000)
    elif kind == "subnormal_d":
        blk[:, 0:208] = _bytes(rng, n * 208).reshape(n, 208)
        _put16(blk[:, 208:210], rng.choice(np.array(F16_SUBNORMALS, np.uint16), size=n))
    elif kind == "max_d":
        blk[:, 0:208] = _bytes(rng, n * 208).reshape(n, 208)
        _put16(blk[:, 208:210], rng.choice(np.array([F16_MAX, F16_MINUS_MAX], np.uint16), size=n))
    elif kind == "neg_zero_d":
        blk[:, 0:208] = _bytes(rng, n * 208).reshape(n, 208)
        _put16(blk[:, 208:210], F16_MINUS_ZERO)
    elif kind == "full_range":               # every byte uniform, d of any sign and exponent
        blk[:, 0:208] = _bytes(rng, n * 208).reshape(n, 208)
        _put16(blk[:, 208:210], _f16_random_normal(rng, n))
    else:
        raise ValueError(kind)
    return blk


def _mix(make, kinds, N, nbe, B, seed):
    rng = np.random.default_rng(seed)
    pick = rng.integers(0, len(kinds), size=N * nbe)
    out = np.empty((N * nbe, B), np.uint8)
    for k, kind in enumerate(kinds):
        idx = np.flatnonzero(pick == k)
        if idx.size:
            out[idx] = make(kind, idx.size, rng)
    return out.reshape(N, nbe * B)


def q6k_rows(N: int, nbe: int, seed: int, kinds=Q6K_KINDS) -> np.ndarray:
    """Raw q6_K rows uint8 [N, nbe*210], each block of a kind drawn from `kinds`."""
    return _mix(q6k_blocks, kinds, N, nbe, 210, seed)


KQ_KINDS = ("max_codes_max_scales_neg", "zero_codes_max_scales_maxd", "subnormal_d",
            "neg_zero_d", "full_range")


def kq_blocks(qtype: int, kind: str, n: int, rng) -> np.ndarray:
    """n raw q4_K / q5_K blocks of one kind (d at byte 0, dmin at 2, scales at 4)."""
    B = BLOCK[qtype]
    blk = np.zeros((n, B), np.uint8)
    if kind == "max_codes_max_scales_neg":   # codes 15 / 31, scales, mins 63, d = dmin = -1
        blk[:, 4:B] = 0xFF
        _put16(blk[:, 0:2], F16_MINUS_ONE)
        _put16(blk[:, 2:4], F16_MINUS_ONE)
    elif kind == "zero_codes_max_scales_maxd":   # codes 0, scales, mins 63, d = dmin = max
        blk[:, 4:16] = 0xFF
        _put16(blk[:, 0:2], F16_MAX)
        _put16(blk[:, 2:4], F16_MAX)
    elif kind == "subnormal_d":
        blk[:, 4:B] = _bytes(rng, n * (B - 4)).reshape(n, B - 4)
        _put16(blk[:, 0:2], rng.choice(np.array(F16_SUBNORMALS, np.uint16), size=n))
        _put16(blk[:, 2:4], _f16_random_normal(rng, n) | 0x8000)
    elif kind == "neg_zero_d":
        blk[:, 4:B] = _bytes(rng, n * (B - 4)).reshape(n, B - 4)
        _put16(blk[:, 0:2], F16_MINUS_ZERO)
        _put16(blk[:, 2:4], F16_ONE)
    elif kind == "full_range":
        blk[:, 4:B] = _bytes(rng, n * (B - 4)).reshape(n, B - 4)
        _put16(blk[:, 0:2], _f16_random_normal(rng, n))
        _put16(blk[:, 2:4], _f16_random_normal(rng, n))
    else:
        raise ValueError(kind)
    return blk


def kq_rows(qtype: int, N: int, nbe: int, seed: int, kinds=KQ_KINDS) -> np.ndarray:
    return _mix(lambda kind, n, rng: kq_blocks(qtype, kind, n, rng), kinds, N, nbe,
                BLOCK[qtype], seed)


# q8 activation planes
PLANE_KINDS = ("all_min", "extremes_max_scale", "full_range")


def q8_plane_edge(kind: str, K: int, nt: int, seed: int):
    """(qs int8 [nt, K], d16 uint16 [nt, K/32]) at the edges of the q8 range."""
    rng = np.random.default_rng(seed)
    if kind == "all_min":                    # every code -128, every scale 1
        qs = np.full((nt, K), -128, np.int8)
        d16 = np.full((nt, K // 32), F16_ONE, np.uint16)
    elif kind == "extremes_max_scale":       # codes -128 / 127, scales +-65504
        qs = rng.choice(np.array([-128, 127], np.int8), size=(nt, K))
        d16 = rng.choice(np.array([F16_MAX, F16_MINUS_MAX], np.uint16), size=(nt, K // 32))
    elif kind == "full_range":               # every int8 code; scales of any sign and
        qs = rng.integers(-128, 128, size=(nt, K)).astype(np.int8)   # exponent, subnormal, 0
        d16 = _f16_random_normal(rng, nt * (K // 32)).reshape(nt, K // 32)
        special = np.array(list(F16_SUBNORMALS) + [0, F16_MINUS_ZERO, F16_MAX], np.uint16)
        mask = rng.random(size=d16.shape) < 0.1
        d16[mask] = rng.choice(special, size=int(mask.sum()))
    else:
        raise ValueError(kind)
    return qs, d16
