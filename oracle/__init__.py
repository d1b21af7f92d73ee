"""The oracle for the q6_K (and q4_K / q5_K) x q8 decode GEMV path -- TEST
INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never calls it and the two
share no code: this wraps the plain scalar C in ``q6k_oracle.c`` and
``kq_oracle.c`` (built with gcc) with numpy-array marshalling and nothing else.

Every function names the page passage it follows in ``q6k_oracle.c``. The
RMSNorm reduction order is the one step the pages leave open; its value is
pinned by closed forms, its last bit is not (see ``rmsnorm``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

__all__ = [
    "RAW", "PAD224", "DPL", "build", "row_stride", "f16_to_f64", "f32_to_f16",
    "decode", "dequant", "repack_dpl", "unpack_dpl", "pad224", "quant_q8",
    "rmsnorm", "swiglu", "subdots", "mmvq", "mmvq_exact",
    "Q4_K", "Q5_K", "kq_block_bytes", "kq_row_stride", "kq_decode", "kq_dequant",
    "kq_repack_dpl", "kq_unpack_dpl", "kq_subdots", "kq_mmvq", "kq_mmvq_exact",
]

RAW, PAD224, DPL = 0, 1, 2
Q4_K, Q5_K = 12, 13          # GGUF type ids

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "q6k_oracle.c"), os.path.join(_HERE, "kq_oracle.c")]
_LIB = os.path.join(_HERE, "liborc.so")
_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-fexcess-precision=standard", "-fopenmp",
           *_SRCS, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f)
                                           for f in _SRCS):
            build()
        lib = ctypes.CDLL(_LIB)
        sig = {
            "orc_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
            "orc_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_row_stride": (_I64, [_INT, _I64]),
            "orc_decode": (_INT, [_INT, _P, _I64, _I64, _P, _P, _P]),
            "orc_dequant": (_INT, [_INT, _P, _I64, _I64, _P]),
            "orc_repack_dpl": (_INT, [_P, _P, _I64, _I64]),
            "orc_unpack_dpl": (_INT, [_P, _P, _I64, _I64]),
            "orc_pad224": (_INT, [_P, _P, _I64, _I64]),
            "orc_quant_q8": (_INT, [_P, _I64, _INT, _P, _P]),
            "orc_rmsnorm": (_INT, [_P, _P, ctypes.c_float, _I64, _INT, _P]),
            "orc_swiglu": (_INT, [_P, _P, _I64, _INT, _P]),
            "orc_subdots": (_INT, [_INT, _P, _I64, _I64, _INT, _P, _P]),
            "orc_mmvq": (_INT, [_INT, _P, _I64, _I64, _INT, _P, _P, _P, _P, _INT]),
            "orc_mmvq_exact": (_INT, [_INT, _P, _I64, _I64, _INT, _P, _P, _P]),
            "orc_kq_block_bytes": (_I64, [_INT]),
            "orc_kq_row_stride": (_I64, [_INT, _INT, _I64]),
            "orc_kq_decode": (_INT, [_INT, _INT, _P, _I64, _I64, _P, _P, _P, _P, _P]),
            "orc_kq_dequant": (_INT, [_INT, _INT, _P, _I64, _I64, _P]),
            "orc_kq_repack_dpl": (_INT, [_INT, _P, _P, _I64, _I64]),
            "orc_kq_unpack_dpl": (_INT, [_INT, _P, _P, _I64, _I64]),
            "orc_kq_subdots": (_INT, [_INT, _INT, _P, _I64, _I64, _INT, _P, _P]),
            "orc_kq_mmvq": (_INT, [_INT, _INT, _P, _I64, _I64, _INT, _P, _P, _P, _P, _INT]),
            "orc_kq_mmvq_exact": (_INT, [_INT, _INT, _P, _I64, _I64, _INT, _P, _P, _P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint8)


def row_stride(layout: int, K: int) -> int:
    s = _load().orc_row_stride(layout, K)
    if s < 0:
        raise ValueError(f"K={K} is not a positive multiple of 256")
    return int(s)


def f16_to_f64(h: int) -> float:
    return float(_load().orc_f16_to_f64(int(h) & 0xFFFF))


def f32_to_f16(f: float) -> int:
    return int(_load().orc_f32_to_f16(float(np.float32(f))))


def decode(layout: int, W, N: int, K: int):
    """-> (q uint8 [N,K] in 0..63, sc int8 [N,K/16], d16 uint16 [N,K/256])."""
    W = _u8(W)
    assert W.size >= N * row_stride(layout, K)
    q = np.empty((N, K), np.uint8)
    sc = np.empty((N, K // 16), np.int8)
    d = np.empty((N, K // 256), np.uint16)
    _check(_load().orc_decode(layout, _ptr(W), N, K, _ptr(q), _ptr(sc), _ptr(d)), "decode")
    return q, sc, d


def dequant(layout: int, W, N: int, K: int) -> np.ndarray:
    W = _u8(W)
    assert W.size >= N * row_stride(layout, K)
    w = np.empty((N, K), np.float64)
    _check(_load().orc_dequant(layout, _ptr(W), N, K, _ptr(w)), "dequant")
    return w


def repack_dpl(raw, N: int, K: int) -> np.ndarray:
    raw = _u8(raw)
    assert raw.size >= N * row_stride(RAW, K)
    out = np.empty(N * row_stride(DPL, K), np.uint8)
    _check(_load().orc_repack_dpl(_ptr(raw), _ptr(out), N, K), "repack_dpl")
    return out


def unpack_dpl(dpl, N: int, K: int) -> np.ndarray:
    dpl = _u8(dpl)
    assert dpl.size >= N * row_stride(DPL, K)
    out = np.empty(N * row_stride(RAW, K), np.uint8)
    _check(_load().orc_unpack_dpl(_ptr(dpl), _ptr(out), N, K), "unpack_dpl")
    return out


def pad224(raw, N: int, K: int) -> np.ndarray:
    raw = _u8(raw)
    assert raw.size >= N * row_stride(RAW, K)
    out = np.empty(N * row_stride(PAD224, K), np.uint8)
    _check(_load().orc_pad224(_ptr(raw), _ptr(out), N, K), "pad224")
    return out


def quant_q8(x) -> tuple[np.ndarray, np.ndarray]:
    """x float32 [nt, K] -> (qs int8 [nt, K], d16 uint16 [nt, K/32])."""
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    nt, K = x.shape
    qs = np.empty((nt, K), np.int8)
    d = np.empty((nt, K // 32), np.uint16)
    _check(_load().orc_quant_q8(_ptr(x), K, nt, _ptr(qs), _ptr(d)), "quant_q8")
    return qs, d


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """x float32 [nt, K], gamma float32 [K] -> y float32 [nt, K]."""
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    nt, K = x.shape
    assert gamma.shape == (K,)
    y = np.empty((nt, K), np.float32)
    _check(_load().orc_rmsnorm(_ptr(x), _ptr(gamma), float(eps), K, nt, _ptr(y)), "rmsnorm")
    return y


def swiglu(g, u) -> np.ndarray:
    """g, u float32 [nt, K] -> y = silu(g) * u float32 [nt, K] (evaluated in fp64, then
    rounded to f32: within an ulp of the exactly rounded value)."""
    g = np.ascontiguousarray(np.atleast_2d(g), dtype=np.float32)
    u = np.ascontiguousarray(np.atleast_2d(u), dtype=np.float32)
    assert g.shape == u.shape
    nt, K = g.shape
    y = np.empty((nt, K), np.float32)
    _check(_load().orc_swiglu(_ptr(g), _ptr(u), K, nt, _ptr(y)), "swiglu")
    return y


def subdots(layout: int, W, N: int, K: int, qs) -> np.ndarray:
    """-> int32 [nt, N, K/16]."""
    W = _u8(W)
    qs = np.ascontiguousarray(np.atleast_2d(qs), dtype=np.int8)
    nt = qs.shape[0]
    assert qs.shape == (nt, K) and W.size >= N * row_stride(layout, K)
    out = np.empty((nt, N, K // 16), np.int32)
    _check(_load().orc_subdots(layout, _ptr(W), N, K, nt, _ptr(qs), _ptr(out)), "subdots")
    return out


def mmvq(layout: int, W, N: int, K: int, qs, d16, nthreads: int = 1):
    """-> (y float64 [nt, N], A float64 [nt, N]) with A = sum of |terms|."""
    W = _u8(W)
    qs = np.ascontiguousarray(np.atleast_2d(qs), dtype=np.int8)
    d16 = np.ascontiguousarray(np.atleast_2d(d16), dtype=np.uint16)
    nt = qs.shape[0]
    assert qs.shape == (nt, K) and d16.shape == (nt, K // 32)
    assert W.size >= N * row_stride(layout, K)
    y = np.empty((nt, N), np.float64)
    A = np.empty((nt, N), np.float64)
    _check(_load().orc_mmvq(layout, _ptr(W), N, K, nt, _ptr(qs), _ptr(d16), _ptr(y),
                            _ptr(A), int(nthreads)), "mmvq")
    return y, A


def mmvq_exact(layout: int, W, N: int, K: int, qs, d16) -> np.ndarray:
    """The exact sum (128-bit integer in units of 2^-48), rounded once to fp64."""
    W = _u8(W)
    qs = np.ascontiguousarray(np.atleast_2d(qs), dtype=np.int8)
    d16 = np.ascontiguousarray(np.atleast_2d(d16), dtype=np.uint16)
    nt = qs.shape[0]
    assert qs.shape == (nt, K) and d16.shape == (nt, K // 32)
    y = np.empty((nt, N), np.float64)
    _check(_load().orc_mmvq_exact(layout, _ptr(W), N, K, nt, _ptr(qs), _ptr(d16), _ptr(y)),
           "mmvq_exact")
    return y


# --- q4_K / q5_K (kq_oracle.c) ------------------------------------------------------

def kq_block_bytes(qtype: int) -> int:
    b = int(_load().orc_kq_block_bytes(qtype))
    if b <= 0:
        raise ValueError(f"unknown k-quant type {qtype}")
    return b


def kq_row_stride(qtype: int, layout: int, K: int) -> int:
    s = _load().orc_kq_row_stride(qtype, layout, K)
    if s < 0:
        raise ValueError(f"type {qtype} layout {layout} K={K}: bad shape")
    return int(s)


def kq_decode(qtype: int, layout: int, W, N: int, K: int):
    """-> (codes uint8 [N,K], sc uint8 [N,K/32], m uint8 [N,K/32], d16 uint16 [N,K/256],
    dmin16 uint16 [N,K/256])."""
    W = _u8(W)
    assert W.size >= N * kq_row_stride(qtype, layout, K)
    q = np.empty((N, K), np.uint8)
    sc = np.empty((N, K // 32), np.uint8)
    m = np.empty((N, K // 32), np.uint8)
    d = np.empty((N, K // 256), np.uint16)
    dm = np.empty((N, K // 256), np.uint16)
    _check(_load().orc_kq_decode(qtype, layout, _ptr(W), N, K, _ptr(q), _ptr(sc), _ptr(m),
                                 _ptr(d), _ptr(dm)), "kq_decode")
    return q, sc, m, d, dm


def kq_dequant(qtype: int, layout: int, W, N: int, K: int) -> np.ndarray:
    W = _u8(W)
    assert W.size >= N * kq_row_stride(qtype, layout, K)
    w = np.empty((N, K), np.float64)
    _check(_load().orc_kq_dequant(qtype, layout, _ptr(W), N, K, _ptr(w)), "kq_dequant")
    return w


def kq_repack_dpl(qtype: int, raw, N: int, K: int) -> np.ndarray:
    raw = _u8(raw)
    assert raw.size >= N * kq_row_stride(qtype, RAW, K)
    out = np.empty(N * kq_row_stride(qtype, DPL, K), np.uint8)
    _check(_load().orc_kq_repack_dpl(qtype, _ptr(raw), _ptr(out), N, K), "kq_repack_dpl")
    return out


def kq_unpack_dpl(qtype: int, dpl, N: int, K: int) -> np.ndarray:
    dpl = _u8(dpl)
    assert dpl.size >= N * kq_row_stride(qtype, DPL, K)
    out = np.empty(N * kq_row_stride(qtype, RAW, K), np.uint8)
    _check(_load().orc_kq_unpack_dpl(qtype, _ptr(dpl), _ptr(out), N, K), "kq_unpack_dpl")
    return out


def kq_subdots(qtype: int, layout: int, W, N: int, K: int, qs) -> np.ndarray:
    """-> int32 [nt, N, K/32]: sum of code * x8 per 32-element sub-block."""
    W = _u8(W)
    qs = np.ascontiguousarray(np.atleast_2d(qs), dtype=np.int8)
    nt = qs.shape[0]
    assert qs.shape == (nt, K) and W.size >= N * kq_row_stride(qtype, layout, K)
    out = np.empty((nt, N, K // 32), np.int32)
    _check(_load().orc_kq_subdots(qtype, layout, _ptr(W), N, K, nt, _ptr(qs), _ptr(out)),
           "kq_subdots")
    return out


def kq_mmvq(qtype: int, layout: int, W, N: int, K: int, qs, d16, nthreads: int = 1):
    """-> (y float64 [nt, N], A float64 [nt, N]) with A = sum of |terms|."""
    W = _u8(W)
    qs = np.ascontiguousarray(np.atleast_2d(qs), dtype=np.int8)
    d16 = np.ascontiguousarray(np.atleast_2d(d16), dtype=np.uint16)
    nt = qs.shape[0]
    assert qs.shape == (nt, K) and d16.shape == (nt, K // 32)
    assert W.size >= N * kq_row_stride(qtype, layout, K)
    y = np.empty((nt, N), np.float64)
    A = np.empty((nt, N), np.float64)
    _check(_load().orc_kq_mmvq(qtype, layout, _ptr(W), N, K, nt, _ptr(qs), _ptr(d16), _ptr(y),
                               _ptr(A), int(nthreads)), "kq_mmvq")
    return y, A


def kq_mmvq_exact(qtype: int, layout: int, W, N: int, K: int, qs, d16) -> np.ndarray:
    W = _u8(W)
    qs = np.ascontiguousarray(np.atleast_2d(qs), dtype=np.int8)
    d16 = np.ascontiguousarray(np.atleast_2d(d16), dtype=np.uint16)
    nt = qs.shape[0]
    assert qs.shape == (nt, K) and d16.shape == (nt, K // 32)
    y = np.empty((nt, N), np.float64)
    _check(_load().orc_kq_mmvq_exact(qtype, layout, _ptr(W), N, K, nt, _ptr(qs), _ptr(d16),
                                     _ptr(y)), "kq_mmvq_exact")
    return y
