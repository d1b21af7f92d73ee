"""GPU parity of the fused RMSNorm -> q8 -> GEMV entry point.

Its outputs must equal those of the producer followed by the GEMV bit for bit
(both sides are the library's, so this pins the fused kernel to the path the other
tests check against the oracle), and they are checked against the oracle directly
on every call: the normalized row within 2 ulp of the oracle's RMSNorm, the q8 plane
bit for bit against the oracle quantizer of that row (and within the block rule of
the oracle chain's), and y against the oracle GEMV on the kernel's own q8 plane.
"""
import numpy as np
import pytest
import torch

import oracle
import q6ksynth
import quantized_decode_gemv_amd as q
from gpu_util import (DEV, check_plane_vs_oracle_chain, check_y_on_plane, dev_f32, dpl_from_raw,
                      say, split_plane)

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def _two_kernel(dpl, xd, gd, eps, N, K, nt):
    xn = torch.empty((nt, K), dtype=torch.float32, device=DEV)
    plane = torch.empty(q.q8_plane_bytes(K, nt), dtype=torch.uint8, device=DEV)
    y = torch.empty((nt, N), dtype=torch.float32, device=DEV)
    q.rmsnorm_quant_q8(xd, gd, eps, xn, plane, K, nt)
    q.mmvq_q6k_q8(dpl, plane, y, N, K, nt)
    torch.cuda.synchronize()
    return y.cpu().numpy(), plane.cpu().numpy(), xn.cpu().numpy()


def _fused(dpl, xd, gd, eps, N, K, nt, with_xn=True):
    """Outputs sit inside sentinel-filled buffers, so a write past them shows."""
    pad = 256
    nq = q.q8_plane_bytes(K, nt)
    qbuf = torch.full((nq + 2 * pad,), SENTINEL, dtype=torch.uint8, device=DEV)
    ybuf = torch.full((nt * N + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
    xbuf = torch.full((nt * K + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
    xn = xbuf[pad:pad + nt * K] if with_xn else None
    q.mmvq_q6k_rmsnorm_q8(dpl, xd, gd, eps, xn, qbuf[pad:pad + nq], ybuf[pad:pad + nt * N],
                          N, K, nt)
    torch.cuda.synchronize()
    qb, yb, xb = qbuf.cpu().numpy(), ybuf.cpu().numpy(), xbuf.cpu().numpy()
    assert np.all(qb[:pad] == SENTINEL) and np.all(qb[pad + nq:] == SENTINEL)
    assert np.all(np.isnan(yb[:pad])) and np.all(np.isnan(yb[pad + nt * N:]))
    assert np.all(np.isnan(xb[:pad])) and np.all(np.isnan(xb[pad + nt * K:]))
    if not with_xn:
        assert np.all(np.isnan(xb))
    return (yb[pad:pad + nt * N].reshape(nt, N), qb[pad:pad + nq],
            xb[pad:pad + nt * K].reshape(nt, K))


def _inputs(N, K, nt, seed):
    raw = q6ksynth.raw_q6k(N, K, seed=seed)
    x = np.stack([q6ksynth.activation("outlier", K, seed + 1 + c) for c in range(nt)])
    g = q6ksynth.gamma(K, seed + 999)
    return raw, x, g


def _check_against_oracle(raw, x, g, eps, y, plane, xn, N, K, nt, what):
    x_or = oracle.rmsnorm(x, g, eps)
    qs_or, d_or = oracle.quant_q8(x_or)
    qs = plane[:nt * K].view(np.int8).reshape(nt, K)
    d = plane[nt * K:].view(np.uint16).reshape(nt, K // 32)
    ulp = np.spacing(np.abs(x_or))
    assert np.all(np.abs(xn - x_or) <= 2 * ulp), f"{what}: normalized row beyond 2 ulp"
    rep = check_plane_vs_oracle_chain(xn, x_or, qs, d, qs_or, d_or, what)
    # y against the oracle GEMV on the kernel's own q8 plane, always
    rep["max_err_over_A"] = check_y_on_plane(y, raw, qs, d, N, K, what)
    return rep


@pytest.mark.parametrize("name,nt", [("attn_v", 1), ("lm_head", 1), ("lm_head", 4)])
def test_fused_workloads(name, nt):
    w = q6ksynth.WORKLOADS[name]
    say(f"fused workload {name} N={w.N} K={w.K} nt={nt}")
    assert q.rmsnorm_mmvq_fused(w.N, w.K, nt) == (nt == 1)
    raw = q6ksynth.weights(w)
    dpl = dpl_from_raw(raw, w.N, w.K)
    x = q6ksynth.activations(w, nt)
    g = q6ksynth.gamma(w.K, q6ksynth.gamma_seed(w))
    xd, gd = dev_f32(x), dev_f32(g)
    y1, p1, xn1 = _fused(dpl, xd, gd, q6ksynth.RMS_EPS, w.N, w.K, nt)
    y2, p2, xn2 = _two_kernel(dpl, xd, gd, q6ksynth.RMS_EPS, w.N, w.K, nt)
    assert np.array_equal(p1, p2)
    assert np.array_equal(xn1.view(np.uint32), xn2.view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    rep = _check_against_oracle(raw, x, g, q6ksynth.RMS_EPS, y1, p1, xn1, w.N, w.K, nt, name)
    say(f"  fused == producer + GEMV bitwise; vs oracle chain: {rep}")


# chunks per lane 1..7 (the fused kernel takes 1..6 with one token), and the
# two-kernel form for several tokens and longer rows
EDGE = ([(nbe, 1) for nbe in (1, 2, 7, 8, 9, 16, 17, 24, 25, 32, 33, 40, 41, 47, 48, 49, 74)]
        + [(nbe, nt) for nbe in (1, 20, 49) for nt in (2, 3, 4, 5)])


@pytest.mark.parametrize("nbe,nt", EDGE)
def test_fused_edges(nbe, nt):
    N, K = 67, 256 * nbe
    assert q.rmsnorm_mmvq_fused(N, K, nt) == (nt == 1 and nbe <= 48)
    raw, x, g = _inputs(N, K, nt, seed=7000 + 10 * nbe + nt)
    dpl = dpl_from_raw(raw, N, K)
    xd, gd = dev_f32(x), dev_f32(g)
    y1, p1, xn1 = _fused(dpl, xd, gd, 1e-6, N, K, nt)
    y2, p2, xn2 = _two_kernel(dpl, xd, gd, 1e-6, N, K, nt)
    assert np.array_equal(p1, p2)
    assert np.array_equal(xn1.view(np.uint32), xn2.view(np.uint32))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    _check_against_oracle(raw, x, g, 1e-6, y1, p1, xn1, N, K, nt, f"nbe={nbe} nt={nt}")


@pytest.mark.parametrize("N", [1, 2, 3, 5, 255, 257, 1023])
@pytest.mark.parametrize("nt", [1, 2])
def test_fused_row_counts_and_no_xn(N, nt):
    K = 5120
    raw, x, g = _inputs(N, K, nt, seed=7500 + 3 * N + nt)
    dpl = dpl_from_raw(raw, N, K)
    xd, gd = dev_f32(x), dev_f32(g)
    y1, p1, _ = _fused(dpl, xd, gd, 0.5, N, K, nt, with_xn=False)
    y2, p2, xn2 = _two_kernel(dpl, xd, gd, 0.5, N, K, nt)
    assert np.array_equal(p1, p2)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    _check_against_oracle(raw, x, g, 0.5, y1, p1, xn2, N, K, nt, f"N={N}")


def test_fused_zero_rows_and_side_stream():
    # an all-zero activation row normalizes to zeros (r = 1/sqrt(eps)): q8 all zero,
    # y exactly zero; on a side stream
    N, K, nt = 300, 1024, 1
    raw, x, g = _inputs(N, K, nt, seed=7700)
    x[0] = 0.0
    dpl = dpl_from_raw(raw, N, K)
    xd, gd = dev_f32(x), dev_f32(g)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    plane = torch.empty(q.q8_plane_bytes(K, nt), dtype=torch.uint8, device=DEV)
    y = torch.empty((nt, N), dtype=torch.float32, device=DEV)
    with torch.cuda.stream(s):
        q.mmvq_q6k_rmsnorm_q8(dpl, xd, gd, 1e-6, None, plane, y, N, K, nt, stream=s)
    s.synchronize()
    yh = y.cpu().numpy()
    qs, d = split_plane(plane, K, nt)
    assert not qs[0].any() and not d[0].any() and not yh[0].any()
    y2, p2, _ = _two_kernel(dpl, xd, gd, 1e-6, N, K, nt)
    assert np.array_equal(plane.cpu().numpy(), p2)
    assert np.array_equal(yh.view(np.uint32), y2.view(np.uint32))
