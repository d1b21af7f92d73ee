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


def check_plane_vs_oracle_chain(y_gpu, y_or, qs, d16, qs_or, d_or, what: str) -> dict:
    """Compare a producer's q8 plane with the oracle chain's, block by block.

    Blocks whose 32 producer outputs equal the oracle's bit for bit must give the
    same q8 bytes (the quantizer is a per-block function of its inputs). The RMSNorm
    reduction order is left open by the pages, so a block holding an output that
    differs in its last bits may differ by at most one code per element and one
    fp16 step in its scale. Returns counts for the report.
    """
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
