"""Test-side helpers for the GPU parity tests: device buffers and oracle runs."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
import quantized_decode_gemv_amd as q

DEV = "cuda:0"
TOL = 1e-5          # |y - y_oracle| <= TOL * sum|terms| (spec bound)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to(DEV)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dpl_from_raw(raw: np.ndarray, N: int, K: int) -> torch.Tensor:
    """Repack on the device (the library's repack) from host raw bytes."""
    raw_d = dev_u8(raw)
    assert raw_d.numel() == q.q6k_raw_bytes(N, K)
    dpl = torch.empty(q.q6k_dpl_bytes(N, K), dtype=torch.uint8, device=DEV)
    q.repack_q6k_dpl(raw_d, dpl, N, K)
    return dpl


def q8_plane(K: int, nt: int) -> torch.Tensor:
    return torch.empty(q.q8_plane_bytes(K, nt), dtype=torch.uint8, device=DEV)


def split_plane(plane: torch.Tensor, K: int, nt: int):
    """Device q8 plane -> (qs int8 [nt, K], d16 uint16 [nt, K/32]) on the host."""
    b = plane.cpu().numpy()
    qs = b[:nt * K].view(np.int8).reshape(nt, K)
    d16 = b[nt * K: nt * K + nt * (K // 32) * 2].view(np.uint16).reshape(nt, K // 32)
    return qs, d16


def make_plane(qs: np.ndarray, d16: np.ndarray) -> torch.Tensor:
    """Host (qs, d16) -> a device q8 plane (for feeding the GEMV oracle-made inputs)."""
    nt, K = qs.shape
    buf = np.concatenate([qs.reshape(-1).view(np.uint8), d16.reshape(-1).view(np.uint8)])
    assert buf.size == q.q8_plane_bytes(K, nt)
    return dev_u8(buf)


def run_mmvq(dpl: torch.Tensor, plane: torch.Tensor, N: int, K: int, nt: int) -> np.ndarray:
    y = torch.full((nt, N), float("nan"), dtype=torch.float32, device=DEV)
    q.mmvq_q6k_q8(dpl, plane, y, N, K, nt)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_y(y: np.ndarray, y_or: np.ndarray, A: np.ndarray, what: str) -> float:
    """Assert the benchmark spec's bound; return the worst err / A."""
    assert y.shape == y_or.shape
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    err = np.abs(y.astype(np.float64) - y_or)
    zero = A == 0
    assert np.all(y[zero] == 0), f"{what}: rows with no terms must be exactly 0"
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, A))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= TOL, f"{what}: max err/A = {worst:.3e} at {np.unravel_index(ratio.argmax(), ratio.shape)}"
    return worst


def check_plane_exact(y_gpu, qs, d16, what: str) -> None:
    """A producer's q8 plane must be the oracle quantizer applied to the producer's
    own y, bit for bit, on every block (the quantizer is a per-block function of its
    32 inputs)."""
    qs_o, d_o = oracle.quant_q8(np.ascontiguousarray(y_gpu, dtype=np.float32))
    bad = np.flatnonzero(np.any(qs.reshape(-1, 32) != qs_o.reshape(-1, 32), axis=1)
                         | (d16.reshape(-1) != d_o.reshape(-1)))
    assert bad.size == 0, (f"{what}: q8 plane differs from the oracle quantizer of the "
                           f"producer's own y in {bad.size} blocks (first {bad[:4]})")


def check_plane_vs_oracle_chain(y_gpu, y_or, qs, d16, qs_or, d_or, what: str) -> dict:
    """Check a producer's q8 plane against the oracle.

    First, bit for bit against the oracle quantizer applied to the producer's own y
    (check_plane_exact). Then against the oracle chain (the oracle quantizer applied
    to the oracle's y), block by block: blocks whose 32 producer outputs equal the
    oracle's bit for bit must give the same q8 bytes; the RMSNorm reduction order
    is left open by the pages, so a block holding an output that differs in its last
    bits may differ by at most one code per element and one fp16 step in its scale.
    Returns counts for the report.
    """
    check_plane_exact(y_gpu, qs, d16, what)
    nt, K = qs.shape
    yb = y_gpu.reshape(nt, K // 32, 32)
    ob = y_or.reshape(nt, K // 32, 32)
    same_in = np.all(yb.view(np.uint32) == ob.view(np.uint32), axis=2)     # [nt, K/32]
    qb, qob = qs.reshape(nt, K // 32, 32), qs_or.reshape(nt, K // 32, 32)
    same_out = np.all(qb == qob, axis=2) & (d16 == d_or)
    assert np.all(same_out[same_in]), f"{what}: q8 differs on a block with identical inputs"
    dq = np.abs(qb.astype(np.int32) - qob.astype(np.int32))
    dd = np.abs(d16.astype(np.int32) - d_or.astype(np.int32))
    assert dq[~same_in].max(initial=0) <= 1 and dd[~same_in].max(initial=0) <= 1, what
    return dict(blocks=int(same_in.size), blocks_inputs_differ=int((~same_in).sum()),
                codes_differ=int((qs != qs_or).sum()))


def oracle_gemv(qtype: int, raw, N: int, K: int, qs, d16):
    """The oracle GEMV (raw rows) of any weight type: (y, A)."""
    if qtype == q.KQ_Q6_K:
        return oracle.mmvq(oracle.RAW, raw, N, K, qs, d16, nthreads=oracle_threads())
    return oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, qs, d16, nthreads=oracle_threads())


def check_y_on_plane(y, raw, qs, d16, N: int, K: int, what: str, qtype: int = None) -> float:
    """y of the GPU's whole chain against the oracle GEMV run on the GPU's own q8
    plane (qs, d16), so the check never depends on the producer matching the oracle
    chain bit for bit. Returns the worst err / A."""
    y_or, A = oracle_gemv(q.KQ_Q6_K if qtype is None else qtype, raw, N, K, qs, d16)
    return check_y(np.asarray(y).reshape(y_or.shape), y_or, A, what)


def swiglu_tol(y_or, g, u):
    """The SwiGLU producer's f32 body g / (1 + expf(-g)) * u (D3-5 §3.2) against the
    oracle's exactly rounded value: expf, 1 + e, the division and the product each
    round once, so 4 ulp; and where expf(-g) overflows f32 (g below about -88.7) the
    body gives g / inf = -0, while the exact value is below |g * u| * e^g < |g * u| *
    2^-128, so an absolute term |g * u| * 2^-126 covers that tail (and any rounding in
    the subnormal range)."""
    y_or = np.asarray(y_or, np.float64)
    gu = np.abs(np.asarray(g, np.float64) * np.asarray(u, np.float64)).reshape(y_or.shape)
    return (4 * np.spacing(np.abs(y_or).astype(np.float32)).astype(np.float64)
            + gu * 2.0 ** -126)
