"""Pins for the oracle's sub-block dots and GEMV (CPU only).

Closed forms (one-hot diagonal probe, full-coverage sum), special cases, brute
force on tiny inputs, the exact 128-bit sum and the raw == padded == dpl invariant.
"""
import numpy as np
import pytest

import oracle
import q6ksynth
from q6k_build import blank, onehot_probe, set_d


@pytest.mark.parametrize("q0", [0, 1, 31, 33, 63])
@pytest.mark.parametrize("nbe,block", [(1, 0), (4, 3)])
def test_onehot_diagonal(q0, nbe, block):
    raw, qs, d16, expect = onehot_probe(q0, nbe=nbe, block=block)
    K = 256 * nbe
    for layout, W in [(oracle.RAW, raw), (oracle.DPL, oracle.repack_dpl(raw, 256, K))]:
        y, _ = oracle.mmvq(layout, W, 256, K, qs, d16)
        assert np.array_equal(y, expect)
        D = oracle.subdots(layout, W, 256, K, qs)
        # column c, row e: only sub-block e//16 of block `block` is non-zero
        for e in (0, 17, 100, 255):
            nz = np.nonzero(D[e, e])[0]
            assert list(nz) == ([16 * block + e // 16] if q0 != 32 else [])
            assert D[e, e, 16 * block + e // 16] == q0 - 32


@pytest.mark.parametrize("nbe", [1, 2, 5, 20, 54, 74])
@pytest.mark.parametrize("nt", [1, 3])
def test_full_coverage_sum_is_K(nbe, nt):
    # every code 33 (weight 1 * 1 * (33 - 32)), every x8 = 1 with scale 1: y = K exactly.
    # A GEMV that skips any unit falls short by an exact multiple of 32 (D4-2 §2).
    K, N = 256 * nbe, 3
    raw = blank(N, nbe, ql=0x11, qh=0xAA, sc=1, d_bits=0x3C00)
    qs = np.ones((nt, K), np.int8)
    d16 = np.full((nt, K // 32), 0x3C00, np.uint16)
    y, A = oracle.mmvq(oracle.DPL, oracle.repack_dpl(raw, N, K), N, K, qs, d16)
    assert np.all(y == K) and np.all(A == K)


def _rand_q8(K, nt, seed):
    x = np.stack([q6ksynth.activation("outlier", K, seed + c) for c in range(nt)])
    return oracle.quant_q8(x)


@pytest.mark.parametrize("case", ["d0", "q32", "sc0", "x0"])
def test_special_cases_give_zero(case):
    N, K, nt = 4, 1024, 2
    raw = q6ksynth.raw_q6k(N, K, seed=11)
    qs, d16 = _rand_q8(K, nt, 50)
    blocks = raw.reshape(N, K // 256, 210)
    if case == "d0":
        blocks[:, :, 208:210] = 0
    elif case == "q32":
        blocks[:, :, :128] = 0
        blocks[:, :, 128:192] = 0xAA
    elif case == "sc0":
        blocks[:, :, 192:208] = 0
    else:
        qs[:] = 0
        d16[:] = 0
    y, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d16)
    assert np.all(y == 0) and np.all(A == 0)


def test_doubling_d_doubles_y_exactly():
    N, K, nt = 5, 2048, 1
    raw = q6ksynth.raw_q6k(N, K, seed=12)
    qs, d16 = _rand_q8(K, nt, 60)
    y1, _ = oracle.mmvq(oracle.RAW, raw, N, K, qs, d16)
    blocks = raw.reshape(N, K // 256, 210)
    d = blocks[:, :, 208:210].copy().view(np.float16)
    assert np.any(d < np.float16(2.0 ** -14)), "want some subnormal scales in the case"
    blocks[:, :, 208:210] = (d * np.float16(2)).view(np.uint8)  # exact in fp16
    y2, _ = oracle.mmvq(oracle.RAW, raw, N, K, qs, d16)
    assert np.array_equal(y2, 2 * y1)


@pytest.mark.parametrize("N,K,nt", [(3, 256, 1), (5, 512, 2), (2, 1024, 3)])
def test_brute_force_dequant_dot(N, K, nt):
    raw = q6ksynth.raw_q6k(N, K, seed=13 + K)
    qs, d16 = _rand_q8(K, nt, 70)
    w = oracle.dequant(oracle.RAW, raw, N, K)                       # [N, K] f64, exact
    d8 = np.array([[oracle.f16_to_f64(h) for h in row] for row in d16])  # [nt, K/32]
    xd = qs.astype(np.float64) * np.repeat(d8, 32, axis=1)          # [nt, K], exact
    brute = xd @ w.T                                                 # [nt, N]
    y, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d16)
    assert np.all(np.abs(y - brute) <= 1e-12 * A)


@pytest.mark.parametrize("N,K,nt", [(16, 2048, 1), (4, 18944, 2)])
def test_fp64_sum_within_bound_of_exact_sum(N, K, nt):
    raw = q6ksynth.raw_q6k(N, K, seed=14)
    qs, d16 = _rand_q8(K, nt, 80)
    y, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d16)
    ex = oracle.mmvq_exact(oracle.RAW, raw, N, K, qs, d16)
    n_terms = K // 16
    assert np.all(np.abs(y - ex) <= n_terms * 2.0 ** -53 * A)
    # and the sums are not trivially zero
    assert np.all(A > 0)


@pytest.mark.parametrize("N,K,nt", [(6, 1024, 1), (3, 13824, 2)])
def test_raw_padded_dpl_bitwise_equal(N, K, nt):
    # D4-4 §2 "Why bitwise survives": same values, same order -> identical outputs.
    raw = q6ksynth.raw_q6k(N, K, seed=15)
    qs, d16 = _rand_q8(K, nt, 90)
    ys = [oracle.mmvq(lay, W, N, K, qs, d16) for lay, W in [
        (oracle.RAW, raw), (oracle.PAD224, oracle.pad224(raw, N, K)),
        (oracle.DPL, oracle.repack_dpl(raw, N, K))]]
    for y, A in ys[1:]:
        assert np.array_equal(y, ys[0][0]) and np.array_equal(A, ys[0][1])


def test_subdots_group_16_consecutive_elements():
    N, K, nt = 4, 1024, 2
    raw = q6ksynth.raw_q6k(N, K, seed=16)
    qs, _ = _rand_q8(K, nt, 95)
    q, _, _ = oracle.decode(oracle.RAW, raw, N, K)
    prod = (q.astype(np.int64)[None] - 32) * qs.astype(np.int64)[:, None, :]   # [nt, N, K]
    expect = prod.reshape(nt, N, K // 16, 16).sum(axis=3)
    D = oracle.subdots(oracle.DPL, oracle.repack_dpl(raw, N, K), N, K, qs)
    assert np.array_equal(D, expect)


def test_mmvq_equals_scaled_subdots_in_order():
    N, K, nt = 3, 2048, 2
    raw = q6ksynth.raw_q6k(N, K, seed=18)
    qs, d16 = _rand_q8(K, nt, 96)
    D = oracle.subdots(oracle.RAW, raw, N, K, qs)
    _, sc, d = oracle.decode(oracle.RAW, raw, N, K)
    y, _ = oracle.mmvq(oracle.RAW, raw, N, K, qs, d16)
    for t in range(nt):
        for r in range(N):
            acc = 0.0
            for j in range(K // 16):
                acc += (oracle.f16_to_f64(d[r, j // 16]) * float(sc[r, j]) *
                        oracle.f16_to_f64(d16[t, j // 2]) * float(D[t, r, j]))
            assert acc == y[t, r]


def test_openmp_rows_match_serial():
    N, K, nt = 64, 5120, 1
    raw = q6ksynth.raw_q6k(N, K, seed=19)
    qs, d16 = _rand_q8(K, nt, 97)
    W = oracle.repack_dpl(raw, N, K)
    y1, A1 = oracle.mmvq(oracle.DPL, W, N, K, qs, d16, nthreads=1)
    y4, A4 = oracle.mmvq(oracle.DPL, W, N, K, qs, d16, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(A1, A4)


def test_set_d_helper_matches_decode():
    raw = blank(1, 2)
    set_d(raw, 0, 1, 0x1234)
    _, _, d = oracle.decode(oracle.RAW, raw, 1, 512)
    assert list(d[0]) == [0, 0x1234]
