"""ctypes marshalling for libq6kdpl.so (see include/q6kdpl.h for the contract)."""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch  # loads the HIP runtime this library then shares (same soname)

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq6kdpl.so")

KQ_Q4_K, KQ_Q5_K, KQ_Q6_K = 12, 13, 14     # weight types (GGUF type ids)
Q6K_MAX_N = 1 << 30
Q6K_MAX_K = 1 << 20
Q6K_MAX_NT = 256

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "q6k_strerror": (ctypes.c_char_p, [_INT]),
    "q6k_version": (ctypes.c_char_p, []),
    "q6k_dpl_row_stride": (_SZ, [_I64]),
    "q6k_dpl_bytes": (_SZ, [_I64, _I64]),
    "q6k_raw_bytes": (_SZ, [_I64, _I64]),
    "q8_plane_bytes": (_SZ, [_I64, _INT]),
    "repack_q6k_dpl_host": (_INT, [_P, _P, _I64, _I64]),
    "unpack_q6k_dpl_host": (_INT, [_P, _P, _I64, _I64]),
    "repack_q6k_dpl": (_INT, [_P, _P, _I64, _I64, _P]),
    "quant_q8": (_INT, [_P, _P, _I64, _INT, _P]),
    "rmsnorm_quant_q8": (_INT, [_P, _P, ctypes.c_float, _P, _P, _I64, _INT, _P]),
    "swiglu_quant_q8": (_INT, [_P, _P, _P, _P, _I64, _INT, _P]),
    "mmvq_q6k_q8": (_INT, [_P, _P, _P, _I64, _I64, _INT, _P]),
    "mmvq_q6k_q8_subdots": (_INT, [_P, _P, _P, _I64, _I64, _INT, _P]),
    "mmvq_q6k_rmsnorm_q8": (_INT, [_P, _P, _P, ctypes.c_float, _P, _P, _P, _I64, _I64, _INT,
                                   _P]),
    "q6k_rmsnorm_mmvq_fused": (_INT, [_I64, _I64, _INT]),
    "kq_block_bytes": (_SZ, [_INT]),
    "kq_dpl_row_stride": (_SZ, [_INT, _I64]),
    "kq_dpl_bytes": (_SZ, [_INT, _I64, _I64]),
    "kq_raw_bytes": (_SZ, [_INT, _I64, _I64]),
    "repack_kq_dpl_host": (_INT, [_INT, _P, _P, _I64, _I64]),
    "unpack_kq_dpl_host": (_INT, [_INT, _P, _P, _I64, _I64]),
    "repack_kq_dpl": (_INT, [_INT, _P, _P, _I64, _I64, _P]),
    "mmvq_kq_q8": (_INT, [_INT, _P, _P, _P, _I64, _I64, _INT, _P]),
    "mmvq_kq_rmsnorm_q8": (_INT, [_INT, _P, _P, _P, ctypes.c_float, _P, _P, _P, _I64, _I64,
                                  _INT, _P]),
    "mmvq_kq_q8_subdots": (_INT, [_INT, _P, _P, _P, _I64, _I64, _INT, _P]),
    "mmvq_kq_gate_up_swiglu_q8": (_INT, [_INT, _P, _P, _P, _P, _P, _I64, _I64, _INT, _P]),
    "kq_gate_up_swiglu_fused": (_INT, [_I64, _I64]),
    "q6k_mmvq_plan": (_INT, [_I64, _I64, _INT, _INT, _P]),
    "kq_mmvq_plan": (_INT, [_INT, _I64, _I64, _INT, _INT, _P]),
}

_lock = threading.Lock()
_lib = None


class Q6kError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        msg = lib().q6k_strerror(code).decode()
        super().__init__(f"{fn}: error {code}: {msg}")


def load(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load the in-tree library; build it first only if it does not exist."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            if not build_if_missing:
                raise FileNotFoundError(f"{LIB_PATH} is not built")
            from . import build as _build
            _build.build()
        dll = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(dll, name)
            fn.restype = res
            fn.argtypes = args
        _lib = dll
        return dll


def lib() -> ctypes.CDLL:
    return _lib if _lib is not None else load()


def _addr(p) -> int | None:
    """Device/host address of a tensor, numpy array or integer (None for NULL)."""
    if p is None:
        return None
    if isinstance(p, torch.Tensor):
        return p.data_ptr()
    if isinstance(p, np.ndarray):
        return p.ctypes.data
    return int(p)


def _need(name: str, t, nbytes: int, device: bool = True) -> None:
    """Refuse a torch tensor that is smaller than the bytes the call touches, not
    contiguous, or on the wrong side of the bus. Integers pass through unchecked."""
    if not isinstance(t, torch.Tensor):
        return
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: buffer holds {have} bytes, the call touches {nbytes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: buffer must be contiguous")
    if device != t.is_cuda:
        raise ValueError(f"{name}: buffer must be on the {'GPU' if device else 'host'}")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _call(name: str, *args) -> None:
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise Q6kError(name, rc)


def q6k_version() -> str:
    return lib().q6k_version().decode()


def q6k_dpl_row_stride(K: int) -> int:
    return int(lib().q6k_dpl_row_stride(K))


def q6k_dpl_bytes(N: int, K: int) -> int:
    return int(lib().q6k_dpl_bytes(N, K))


def q6k_raw_bytes(N: int, K: int) -> int:
    return int(lib().q6k_raw_bytes(N, K))


def q8_plane_bytes(K: int, nt: int) -> int:
    return int(lib().q8_plane_bytes(K, nt))


def repack_q6k_dpl_host(raw, dpl, N: int, K: int) -> None:
    _need("raw", raw, q6k_raw_bytes(N, K), device=False)
    _need("dpl", dpl, q6k_dpl_bytes(N, K), device=False)
    _call("repack_q6k_dpl_host", _addr(raw), _addr(dpl), N, K)


def unpack_q6k_dpl_host(dpl, raw, N: int, K: int) -> None:
    _need("dpl", dpl, q6k_dpl_bytes(N, K), device=False)
    _need("raw", raw, q6k_raw_bytes(N, K), device=False)
    _call("unpack_q6k_dpl_host", _addr(dpl), _addr(raw), N, K)


def repack_q6k_dpl(raw_dev, dpl_dev, N: int, K: int, stream=None) -> None:
    _need("raw_dev", raw_dev, q6k_raw_bytes(N, K))
    _need("dpl_dev", dpl_dev, q6k_dpl_bytes(N, K))
    _call("repack_q6k_dpl", _addr(raw_dev), _addr(dpl_dev), N, K, _stream(stream))


def quant_q8(x, q8, K: int, nt: int, stream=None) -> None:
    _need("x", x, 4 * K * max(nt, 0))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _call("quant_q8", _addr(x), _addr(q8), K, nt, _stream(stream))


def rmsnorm_quant_q8(x, gamma, eps: float, y, q8, K: int, nt: int, stream=None) -> None:
    _need("x", x, 4 * K * max(nt, 0))
    _need("gamma", gamma, 4 * K)
    _need("y", y, 4 * K * max(nt, 0))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _call("rmsnorm_quant_q8", _addr(x), _addr(gamma), float(eps), _addr(y), _addr(q8), K, nt,
          _stream(stream))


def swiglu_quant_q8(g, u, y, q8, K: int, nt: int, stream=None) -> None:
    _need("g", g, 4 * K * max(nt, 0))
    _need("u", u, 4 * K * max(nt, 0))
    _need("y", y, 4 * K * max(nt, 0))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _call("swiglu_quant_q8", _addr(g), _addr(u), _addr(y), _addr(q8), K, nt, _stream(stream))


def mmvq_q6k_q8(w_dpl, q8, y, N: int, K: int, nt: int, stream=None) -> None:
    _need("w_dpl", w_dpl, q6k_dpl_bytes(N, K))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _need("y", y, 4 * max(N, 0) * max(nt, 0))
    _call("mmvq_q6k_q8", _addr(w_dpl), _addr(q8), _addr(y), N, K, nt, _stream(stream))


def mmvq_q6k_rmsnorm_q8(w_dpl, x, gamma, eps: float, xn, q8, y, N: int, K: int, nt: int,
                        stream=None) -> None:
    _need("w_dpl", w_dpl, q6k_dpl_bytes(N, K))
    _need("x", x, 4 * K * max(nt, 0))
    _need("gamma", gamma, 4 * K)
    if xn is not None:
        _need("xn", xn, 4 * K * max(nt, 0))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _need("y", y, 4 * max(N, 0) * max(nt, 0))
    _call("mmvq_q6k_rmsnorm_q8", _addr(w_dpl), _addr(x), _addr(gamma), float(eps), _addr(xn),
          _addr(q8), _addr(y), N, K, nt, _stream(stream))


def rmsnorm_mmvq_fused(N: int, K: int, nt: int) -> bool:
    rc = lib().q6k_rmsnorm_mmvq_fused(N, K, nt)
    if rc < 0:
        raise Q6kError("q6k_rmsnorm_mmvq_fused", rc)
    return bool(rc)


def mmvq_q6k_q8_subdots(w_dpl, q8, dots, N: int, K: int, nt: int, stream=None) -> None:
    _need("w_dpl", w_dpl, q6k_dpl_bytes(N, K))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _need("dots", dots, 4 * max(N, 0) * max(nt, 0) * max(K // 16, 0))
    _call("mmvq_q6k_q8_subdots", _addr(w_dpl), _addr(q8), _addr(dots), N, K, nt,
          _stream(stream))


def mmvq_plan(N: int, K: int, nt: int, num_cu: int, qtype: int = 14) -> dict:
    out = (ctypes.c_int32 * 6)()
    _call("kq_mmvq_plan", qtype, N, K, nt, num_cu, ctypes.addressof(out))
    # act_mode: 0 activation operands re-read per row, 1 held in registers ("hoist"),
    # 2 staged in LDS once per workgroup
    # kind: 0 generic stepping kernel, 1 one wave per row, 2 rows shared by the
    # workgroup's four waves (cpl then counts chunks per thread of the 256), 3 two rows
    # per wave sharing the last chunk slot, 4 16-row tiles on the int8 matrix cores
    return dict(grid=out[0], cpl=out[1], unrolled=out[2] >= 1, shared=out[2] == 2,
                paired=out[2] == 3, tiles=out[2] == 4, kind=out[2], hoist=out[3] == 1,
                act_mode=out[3], launches=out[4], depth=out[5])


# --- by weight type (q4_K, q5_K, q6_K) ---------------------------------------------

def kq_block_bytes(qtype: int) -> int:
    return int(lib().kq_block_bytes(qtype))


def kq_dpl_row_stride(qtype: int, K: int) -> int:
    return int(lib().kq_dpl_row_stride(qtype, K))


def kq_dpl_bytes(qtype: int, N: int, K: int) -> int:
    return int(lib().kq_dpl_bytes(qtype, N, K))


def kq_raw_bytes(qtype: int, N: int, K: int) -> int:
    return int(lib().kq_raw_bytes(qtype, N, K))


def repack_kq_dpl_host(qtype: int, raw, dpl, N: int, K: int) -> None:
    _need("raw", raw, kq_raw_bytes(qtype, N, K), device=False)
    _need("dpl", dpl, kq_dpl_bytes(qtype, N, K), device=False)
    _call("repack_kq_dpl_host", qtype, _addr(raw), _addr(dpl), N, K)


def unpack_kq_dpl_host(qtype: int, dpl, raw, N: int, K: int) -> None:
    _need("dpl", dpl, kq_dpl_bytes(qtype, N, K), device=False)
    _need("raw", raw, kq_raw_bytes(qtype, N, K), device=False)
    _call("unpack_kq_dpl_host", qtype, _addr(dpl), _addr(raw), N, K)


def repack_kq_dpl(qtype: int, raw_dev, dpl_dev, N: int, K: int, stream=None) -> None:
    _need("raw_dev", raw_dev, kq_raw_bytes(qtype, N, K))
    _need("dpl_dev", dpl_dev, kq_dpl_bytes(qtype, N, K))
    _call("repack_kq_dpl", qtype, _addr(raw_dev), _addr(dpl_dev), N, K, _stream(stream))


def mmvq_kq_q8(qtype: int, w_dpl, q8, y, N: int, K: int, nt: int, stream=None) -> None:
    _need("w_dpl", w_dpl, kq_dpl_bytes(qtype, N, K))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _need("y", y, 4 * max(N, 0) * max(nt, 0))
    _call("mmvq_kq_q8", qtype, _addr(w_dpl), _addr(q8), _addr(y), N, K, nt, _stream(stream))


def mmvq_kq_rmsnorm_q8(qtype: int, w_dpl, x, gamma, eps: float, xn, q8, y, N: int, K: int,
                       nt: int, stream=None) -> None:
    _need("w_dpl", w_dpl, kq_dpl_bytes(qtype, N, K))
    _need("x", x, 4 * K * max(nt, 0))
    _need("gamma", gamma, 4 * K)
    if xn is not None:
        _need("xn", xn, 4 * K * max(nt, 0))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _need("y", y, 4 * max(N, 0) * max(nt, 0))
    _call("mmvq_kq_rmsnorm_q8", qtype, _addr(w_dpl), _addr(x), _addr(gamma), float(eps),
          _addr(xn), _addr(q8), _addr(y), N, K, nt, _stream(stream))


def mmvq_kq_q8_subdots(qtype: int, w_dpl, q8, dots, N: int, K: int, nt: int,
                       stream=None) -> None:
    per_row = K // 16 if qtype == KQ_Q6_K else K // 32
    _need("w_dpl", w_dpl, kq_dpl_bytes(qtype, N, K))
    _need("q8", q8, q8_plane_bytes(K, nt))
    _need("dots", dots, 4 * max(N, 0) * max(nt, 0) * max(per_row, 0))
    _call("mmvq_kq_q8_subdots", qtype, _addr(w_dpl), _addr(q8), _addr(dots), N, K, nt,
          _stream(stream))


def mmvq_kq_gate_up_swiglu_q8(qtype: int, w_gu, q8_in, gu, y, q8_out, Nh: int, K: int,
                              nt: int = 1, stream=None) -> None:
    _need("w_gu", w_gu, kq_dpl_bytes(qtype, 2 * Nh, K))
    _need("q8_in", q8_in, q8_plane_bytes(K, 1))
    _need("gu", gu, 8 * max(Nh, 0))
    if y is not None:
        _need("y", y, 4 * max(Nh, 0))
    _need("q8_out", q8_out, q8_plane_bytes(Nh, 1))
    _call("mmvq_kq_gate_up_swiglu_q8", qtype, _addr(w_gu), _addr(q8_in), _addr(gu), _addr(y),
          _addr(q8_out), Nh, K, nt, _stream(stream))


def gate_up_swiglu_fused(Nh: int, K: int) -> bool:
    rc = lib().kq_gate_up_swiglu_fused(Nh, K)
    if rc < 0:
        raise Q6kError("kq_gate_up_swiglu_fused", rc)
    return bool(rc)
