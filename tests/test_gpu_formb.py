"""GPU parity of Form B (gate+up GEMV, SwiGLU and q8 of one token in one call).

Its outputs must equal mmvq_kq_q8 followed by swiglu_quant_q8 bit for bit, and each
is checked against the oracle directly: gu against the oracle GEMV, y against the
oracle SwiGLU of the returned gate and up halves (4 ulp, the f32 body's roundings),
and the q8 plane bit for bit against the oracle quantizer of the returned y. Writes
outside the outputs are caught by sentinels."""
import numpy as np
import pytest
import torch

import oracle
import q6ksynth
import quantized_decode_gemv_amd as q
from gpu_util import (DEV, check_plane_exact, check_y, dev_u8, make_plane, oracle_threads, say,
                      swiglu_tol)

pytestmark = pytest.mark.gpu

NAMES = {q.KQ_Q4_K: "q4_K", q.KQ_Q5_K: "q5_K", q.KQ_Q6_K: "q6_K"}
PAD = 256


def _weights(qtype, N, K, seed):
    raw = (q6ksynth.raw_q6k(N, K, seed) if qtype == q.KQ_Q6_K
           else q6ksynth.raw_kq(qtype, N, K, seed))
    dpl = torch.empty(q.kq_dpl_bytes(qtype, N, K), dtype=torch.uint8, device=DEV)
    q.repack_kq_dpl(qtype, dev_u8(raw), dpl, N, K)
    return raw, dpl


def _oracle_gemv(qtype, raw, N, K, qs, d):
    if qtype == q.KQ_Q6_K:
        return oracle.mmvq(oracle.RAW, raw, N, K, qs, d, nthreads=oracle_threads())
    return oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, qs, d, nthreads=oracle_threads())


def _form_b(qtype, dpl, plane, Nh, K, with_y):
    gbuf = torch.full((2 * Nh + 2 * PAD,), float("nan"), dtype=torch.float32, device=DEV)
    ybuf = torch.full((Nh + 2 * PAD,), float("nan"), dtype=torch.float32, device=DEV)
    nq = q.q8_plane_bytes(Nh, 1)
    qbuf = torch.full((nq + 2 * PAD,), 0xA5, dtype=torch.uint8, device=DEV)
    y = ybuf[PAD:PAD + Nh] if with_y else None
    q.mmvq_kq_gate_up_swiglu_q8(qtype, dpl, plane, gbuf[PAD:PAD + 2 * Nh], y,
                                qbuf[PAD:PAD + nq], Nh, K)
    torch.cuda.synchronize()
    g, yb, qb = gbuf.cpu().numpy(), ybuf.cpu().numpy(), qbuf.cpu().numpy()
    assert np.all(np.isnan(g[:PAD])) and np.all(np.isnan(g[PAD + 2 * Nh:]))
    assert np.all(np.isnan(yb[:PAD])) and np.all(np.isnan(yb[PAD + Nh:]))
    assert np.all(qb[:PAD] == 0xA5) and np.all(qb[PAD + nq:] == 0xA5)
    if not with_y:
        assert np.all(np.isnan(yb))
    return g[PAD:PAD + 2 * Nh], yb[PAD:PAD + Nh], qb[PAD:PAD + nq]


def _split(qtype, dpl, plane, Nh, K):
    gu = torch.empty(2 * Nh, dtype=torch.float32, device=DEV)
    y = torch.empty(Nh, dtype=torch.float32, device=DEV)
    p = torch.empty(q.q8_plane_bytes(Nh, 1), dtype=torch.uint8, device=DEV)
    q.mmvq_kq_q8(qtype, dpl, plane, gu, 2 * Nh, K, 1)
    q.swiglu_quant_q8(gu[:Nh], gu[Nh:], y, p, Nh, 1)
    torch.cuda.synchronize()
    return gu.cpu().numpy(), y.cpu().numpy(), p.cpu().numpy()


CASES = [(t, Nh, K) for t in (q.KQ_Q4_K, q.KQ_Q5_K, q.KQ_Q6_K)
         for Nh, K in [(32, 256), (64, 1024), (96, 5120), (416, 2048), (1024, 256 * 48),
                       (64, 256 * 49), (13824, 5120)]]


@pytest.mark.parametrize("qtype,Nh,K", CASES, ids=lambda v: str(v))
def test_form_b_equals_gemv_then_swiglu(qtype, Nh, K):
    say(f"form B {NAMES[qtype]} Nh={Nh} K={K} fused={q.gate_up_swiglu_fused(Nh, K)}")
    assert q.gate_up_swiglu_fused(Nh, K) == (K <= 12288)
    raw, dpl = _weights(qtype, 2 * Nh, K, seed=Nh + K + qtype)
    x = q6ksynth.activation("outlier", K, 31 + Nh)[None]
    qs, d = oracle.quant_q8(x)
    plane = make_plane(qs, d)
    ys = {}
    for with_y in (True, False):
        g1, y1, p1 = _form_b(qtype, dpl, plane, Nh, K, with_y)
        g2, y2, p2 = _split(qtype, dpl, plane, Nh, K)
        assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))
        assert np.array_equal(p1, p2)
        if with_y:
            assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
            ys["y"] = y1
    y1 = ys["y"]
    # gu against the oracle GEMV (from the oracle's own inputs)
    y_or, A = _oracle_gemv(qtype, raw, 2 * Nh, K, qs, d)
    check_y(g1[None], y_or, A, f"form B gu {NAMES[qtype]}")
    # y against the oracle SwiGLU of the kernel's own gate and up totals
    sw_or = oracle.swiglu(g1[None, :Nh], g1[None, Nh:])[0]
    tol = swiglu_tol(sw_or, g1[:Nh], g1[Nh:])
    assert np.all(np.abs(y1.astype(np.float64) - sw_or) <= tol), "form B y"
    # the q8 plane against the oracle quantizer of the kernel's own y, bit for bit
    check_plane_exact(y1[None], p1[:Nh].view(np.int8)[None], p1[Nh:].view(np.uint16)[None],
                      f"form B q8 {NAMES[qtype]}")
    say(f"  gu, y and q8 against the oracle; y bit-equal fraction {np.mean(y1 == sw_or):.4f}")


def test_form_b_zero_gate_rows_give_zero_block():
    # gate rows with d = 0 make gate outputs exactly 0, so silu(0) * u = 0: the q8
    # block is all zero with scale 0
    qtype, Nh, K = q.KQ_Q4_K, 64, 1024
    raw = q6ksynth.raw_kq(qtype, 2 * Nh, K, seed=3)
    blocks = raw.reshape(2 * Nh, K // 256, 144)
    blocks[:32, :, 0:4] = 0              # d = dmin = 0 on the first 32 gate rows
    dpl = torch.empty(q.kq_dpl_bytes(qtype, 2 * Nh, K), dtype=torch.uint8, device=DEV)
    q.repack_kq_dpl(qtype, dev_u8(blocks.reshape(2 * Nh, -1)), dpl, 2 * Nh, K)
    qs, d = oracle.quant_q8(q6ksynth.activation("normal", K, 4)[None])
    g, y, p = _form_b(qtype, dpl, make_plane(qs, d), Nh, K, True)
    assert not g[:32].any() and not y[:32].any()
    assert not p[:32].any() and p[Nh:Nh + 2].view(np.uint16)[0] == 0
    assert p[32:64].any()
