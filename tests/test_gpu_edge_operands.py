"""Operands at the edges of their ranges: negative, subnormal, largest finite and
negative-zero fp16 scales; q6_K sub-block scales -128 / -1 / 0 / 127 and codes 0 /
63; q4_K / q5_K scales and mins 63 and codes 0 / 15 / 31; q8 codes -128 / 127 with
block scales of either sign, subnormal, largest finite and zero.

CPU tests pin the oracle on these operands by closed forms worked by hand and by
its exact 128-bit sum. GPU tests compare every GEMV kind (one wave per row at 1 and
3 chunks per lane, row pairs, rows shared by a workgroup, operands staged in LDS,
the generic long-row kernel) and the fused RMSNorm -> q8 -> GEMV and Form B kernels
with the oracle: the integer sub-block dots bit for bit, y within the bound.

The q6_K extreme sub-block dot is D = 16 * (0 - 32) * (-128) = 65536 = 2^16, and
with scale -128 the product sc * D = -2^23 sits exactly at the edge of the 24-bit
multiply the kernels use; a row made only of such sub-blocks has the closed form
y = -2^23 * (K / 16) (d = 1, q8 scales 1)."""
import numpy as np
import pytest
import torch

import oracle
import q6ksynth
import quantized_decode_gemv_amd as q
from edge_build import (KQ_KINDS, PLANE_KINDS, Q6K_KINDS, kq_rows, q6k_rows, q8_plane_edge)
from gpu_util import (DEV, check_y, check_y_on_plane, dev_f32, dev_u8, make_plane,
                      oracle_threads, say, split_plane)

Q4, Q5, Q6 = 12, 13, 14
NAMES = {Q4: "q4_K", Q5: "q5_K", Q6: "q6_K"}


def _oracle_y(qtype, raw, N, K, qs, d16):
    if qtype == Q6:
        return oracle.mmvq(oracle.RAW, raw, N, K, qs, d16, nthreads=oracle_threads())
    return oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, qs, d16, nthreads=oracle_threads())


def _oracle_exact(qtype, raw, N, K, qs, d16):
    if qtype == Q6:
        return oracle.mmvq_exact(oracle.RAW, raw, N, K, qs, d16)
    return oracle.kq_mmvq_exact(qtype, oracle.RAW, raw, N, K, qs, d16)


def _rows(qtype, N, nbe, seed, kinds=None):
    if qtype == Q6:
        return q6k_rows(N, nbe, seed, kinds or Q6K_KINDS)
    return kq_rows(qtype, N, nbe, seed, kinds or KQ_KINDS)


# --- the oracle on edge operands (CPU) ----------------------------------------------

@pytest.mark.parametrize("nbe", [1, 4, 20])
def test_oracle_q6k_min_scale_closed_form(nbe):
    """Codes 0, scale -128, d = 1, q8 codes -128, scales 1: every sub-block dot is
    16 * (-32) * (-128) = 65536 and every term -128 * 65536 = -2^23, so
    y = -2^23 * K / 16 exactly."""
    K = 256 * nbe
    raw = q6k_rows(3, nbe, 1, kinds=("min_codes_min_scale",))
    qs, d16 = q8_plane_edge("all_min", K, 2, 2)
    assert np.all(oracle.subdots(oracle.RAW, raw, 3, K, qs) == 65536)
    y, A = oracle.mmvq(oracle.RAW, raw, 3, K, qs, d16)
    assert np.all(y == -(2.0 ** 23) * (K // 16)) and np.all(A == -y)
    assert np.all(oracle.mmvq_exact(oracle.RAW, raw, 3, K, qs, d16) == y)


@pytest.mark.parametrize("nbe", [1, 4])
def test_oracle_q6k_max_codes_negative_d_closed_form(nbe):
    """Codes 63, scale 127, d = -1, q8 codes -128, scales 1: D = 16 * 31 * (-128) =
    -63488 and each term (-1) * 127 * (-63488) = 8062976, so y = 8062976 * K / 16."""
    K = 256 * nbe
    raw = q6k_rows(2, nbe, 1, kinds=("max_codes_max_scale_neg_d",))
    qs, d16 = q8_plane_edge("all_min", K, 1, 2)
    assert np.all(oracle.subdots(oracle.RAW, raw, 2, K, qs) == -63488)
    y, _ = oracle.mmvq(oracle.RAW, raw, 2, K, qs, d16)
    assert np.all(y == 8062976.0 * (K // 16))


@pytest.mark.parametrize("qtype,per_sub", [(Q4, 63 * (32 * 15 * 128 - 32 * 128)),
                                           (Q5, 63 * (32 * 31 * 128 - 32 * 128))],
                         ids=["q4_K", "q5_K"])
def test_oracle_kq_max_codes_negative_scales_closed_form(qtype, per_sub):
    """Codes 15 (q4_K) / 31 (q5_K), scales and mins 63, d = dmin = -1, q8 codes -128
    with scales 1: per 32-element sub-block Dq = 32 * c * (-128), Sx = 32 * (-128) and
    d * sc * Dq - dmin * m * Sx = 63 * (32 * c * 128 - 32 * 128), so
    y = that * K / 32."""
    nbe = 4
    K = 256 * nbe
    raw = kq_rows(qtype, 2, nbe, 1, kinds=("max_codes_max_scales_neg",))
    qs, d16 = q8_plane_edge("all_min", K, 1, 2)
    y, _ = oracle.kq_mmvq(qtype, oracle.RAW, raw, 2, K, qs, d16)
    assert np.all(y == float(per_sub) * (K // 32))


@pytest.mark.parametrize("qtype", [Q4, Q5, Q6], ids=lambda t: NAMES[t])
@pytest.mark.parametrize("plane", PLANE_KINDS)
def test_oracle_edge_rows_within_bound_of_exact_sum(qtype, plane):
    """The fp64 oracle on mixed edge rows stays within n * 2^-53 * sum|T| of the exact
    128-bit sum (n terms per output, each rounding once)."""
    N, nbe, nt = 24, 8, 2
    K = 256 * nbe
    raw = _rows(qtype, N, nbe, 11)
    qs, d16 = q8_plane_edge(plane, K, nt, 12)
    y, A = _oracle_y(qtype, raw, N, K, qs, d16)
    ex = _oracle_exact(qtype, raw, N, K, qs, d16)
    nterms = (K // 16) if qtype == Q6 else 2 * (K // 32)
    assert np.all(np.abs(y - ex) <= nterms * 2.0 ** -53 * A)


# --- the HIP path on edge operands (GPU) ---------------------------------------------

def _dpl(qtype, raw, N, K):
    W = torch.empty(q.kq_dpl_bytes(qtype, N, K), dtype=torch.uint8, device=DEV)
    q.repack_kq_dpl(qtype, dev_u8(raw), W, N, K)
    return W


def _gemv(qtype, W, qs, d16, N, K, nt):
    y = torch.full((nt, N), float("nan"), dtype=torch.float32, device=DEV)
    q.mmvq_kq_q8(qtype, W, make_plane(qs, d16), y, N, K, nt)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# (N, K, nt) per GEMV kind: one wave per row at 1 and 3 chunks per lane (q6_K: 15 rows,
# below one tile); row pairs; rows shared by a workgroup's waves; q6_K operands staged
# in LDS (11 chunks per lane, enough rows for one wave per row); the generic long-row
# kernel; q6_K matrix-core tiles
SHAPES = [("rows-cpl1", 64, 1024, 1), ("rows-cpl3", 15, 5120, 3), ("pairs", 4099, 5120, 2),
          ("shared", 2999, 18944, 1), ("shared-nt2", 1500, 13824, 2),
          ("lds", 8192, 256 * 88, 1), ("long", 67, 256 * 100, 2),
          ("tiles", 16 * 12 * 256 + 3, 5120, 4)]


# (q4_K / q5_K long rows at one token are shared by a workgroup instead of staged; the
# tiles are q6_K's)
EDGE_CASES = [(t,) + s for t in (Q6, Q4, Q5) for s in SHAPES
              if t == Q6 or s[0] not in ("lds", "tiles")]


@pytest.mark.gpu
@pytest.mark.parametrize("qtype,kind,N,K,nt", EDGE_CASES,
                         ids=[f"{NAMES[c[0]]}-{c[1]}" for c in EDGE_CASES])
def test_edge_gemv_every_kind(qtype, kind, N, K, nt):
    plan = q.mmvq_plan(N, K, nt, 256, qtype)
    say(f"edge {NAMES[qtype]} {kind} N={N} K={K} nt={nt}: plan {plan}")
    expect = {"pairs": "paired", "shared": "shared", "shared-nt2": "shared",
              "tiles": "tiles"}.get(kind)
    if expect:
        assert plan[expect]
    if kind == "lds":
        assert plan["act_mode"] == 2 and not plan["shared"]
    if kind == "long":
        assert not plan["unrolled"]
    raw = _rows(qtype, N, K // 256, 100 + N + qtype)
    W = _dpl(qtype, raw, N, K)
    for i, pk in enumerate(PLANE_KINDS):
        qs, d16 = q8_plane_edge(pk, K, nt, 200 + i)
        y = _gemv(qtype, W, qs, d16, N, K, nt)
        y_or, A = _oracle_y(qtype, raw, N, K, qs, d16)
        worst = check_y(y, y_or, A, f"{NAMES[qtype]} {kind} plane {pk}")
        say(f"  plane {pk}: max err/A = {worst:.3e}")


@pytest.mark.gpu
@pytest.mark.parametrize("qtype", [Q6, Q4, Q5], ids=lambda t: NAMES[t])
@pytest.mark.parametrize("N,K,nt", [(37, 5120, 2), (5, 256 * 100, 3)])
def test_edge_subdots_bit_exact(qtype, N, K, nt):
    raw = _rows(qtype, N, K // 256, 300 + N + qtype)
    W = _dpl(qtype, raw, N, K)
    per = K // 16 if qtype == Q6 else K // 32
    for i, pk in enumerate(PLANE_KINDS):
        qs, d16 = q8_plane_edge(pk, K, nt, 400 + i)
        dots = torch.zeros((nt, N, per), dtype=torch.int32, device=DEV)
        q.mmvq_kq_q8_subdots(qtype, W, make_plane(qs, d16), dots, N, K, nt)
        torch.cuda.synchronize()
        exp = (oracle.subdots(oracle.RAW, raw, N, K, qs) if qtype == Q6
               else oracle.kq_subdots(qtype, oracle.RAW, raw, N, K, qs))
        assert np.array_equal(dots.cpu().numpy(), exp), f"{NAMES[qtype]} plane {pk}"


@pytest.mark.gpu
@pytest.mark.parametrize("nbe", [1, 4, 20, 74])
def test_edge_q6k_scale_times_dot_at_2_pow_23(nbe):
    """The closed form y = -2^23 * K / 16 on the GPU, bit for bit, for one and four
    tokens (the rows at one wave per row, row pairs or shared rows)."""
    K = 256 * nbe
    for N, nt in [(67, 1), (4097, 4)]:
        raw = q6k_rows(N, nbe, 1, kinds=("min_codes_min_scale",))
        W = _dpl(Q6, raw, N, K)
        qs, d16 = q8_plane_edge("all_min", K, nt, 2)
        y = _gemv(Q6, W, qs, d16, N, K, nt)
        assert np.all(y == np.float32(-(2.0 ** 23) * (K // 16))), (N, nt, np.unique(y)[:4])


@pytest.mark.gpu
@pytest.mark.parametrize("qtype", [Q6, Q4, Q5], ids=lambda t: NAMES[t])
def test_edge_fused_rmsnorm_and_form_b(qtype):
    """The fused RMSNorm -> q8 -> GEMV kernel and Form B on edge weight rows, against
    the oracle GEMV on each kernel's own q8 plane."""
    N, K = 4096, 5120
    raw = _rows(qtype, N, K // 256, 500 + qtype)
    W = _dpl(qtype, raw, N, K)
    x = q6ksynth.activation("outlier", K, 501)[None]
    g = q6ksynth.gamma(K, 502)
    plane = torch.empty(q.q8_plane_bytes(K, 1), dtype=torch.uint8, device=DEV)
    y = torch.empty((1, N), dtype=torch.float32, device=DEV)
    q.mmvq_kq_rmsnorm_q8(qtype, W, dev_f32(x), dev_f32(g), q6ksynth.RMS_EPS, None, plane, y,
                         N, K, 1)
    torch.cuda.synchronize()
    qs, d = split_plane(plane, K, 1)
    check_y_on_plane(y.cpu().numpy(), raw, qs, d, N, K, "edge fused", qtype=qtype)
    # Form B: the 4096 rows as 2048 gate rows and 2048 up rows (a q8 row of ordinary
    # scale, so the SwiGLU of the totals stays finite)
    Nh = N // 2
    qs2, d2 = oracle.quant_q8(q6ksynth.activation("outlier", K, 503)[None])
    gu = torch.empty(N, dtype=torch.float32, device=DEV)
    out = torch.empty(q.q8_plane_bytes(Nh, 1), dtype=torch.uint8, device=DEV)
    q.mmvq_kq_gate_up_swiglu_q8(qtype, W, make_plane(qs2, d2), gu, None, out, Nh, K)
    torch.cuda.synchronize()
    y_or, A = _oracle_y(qtype, raw, N, K, qs2, d2)
    check_y(gu.cpu().numpy()[None], y_or, A, "edge form B gu")
