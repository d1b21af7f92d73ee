"""Pins for the oracle's fp16 conversion, q8 quantizer and RMSNorm (CPU only)."""
import numpy as np
import pytest

import oracle
from golden_io import q8_cases


@pytest.mark.parametrize("case", q8_cases(), ids=lambda c: c[0])
def test_quant_closed_form(case):
    # D3-5 §3.2 per-32-block body; hand-worked cases in tests/golden/q8_closed_form.txt
    _, x, q, d16 = case
    qs, d = oracle.quant_q8(x[None, :])
    assert np.array_equal(qs[0], q)
    assert int(d[0, 0]) == d16


def test_quant_ties_case_code_sum():
    _, x, q, _ = q8_cases()[0]
    qs, _ = oracle.quant_q8(x[None, :])
    assert int(qs.astype(np.int32).sum()) == 255


# IEEE 754 binary16 textbook values.
F16_KNOWN = [
    (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (65519.0, 0x7BFF),
    (65520.0, 0x7C00), (1e9, 0x7C00), (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000),
    (3 * 2.0 ** -25, 0x0002), (2.0 ** -14, 0x0400), (0.1, 0x2E66), (1 / 3, 0x3555),
    (-0.0, 0x8000), (0.0, 0x0000), (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02),
]


@pytest.mark.parametrize("v,bits", F16_KNOWN)
def test_f16_known_values(v, bits):
    assert oracle.f32_to_f16(v) == bits


def test_f16_exhaustive_round_trip():
    for h in range(0x10000):
        e = (h >> 10) & 31
        if e == 31 and (h & 1023):
            continue                       # NaN payloads
        v = oracle.f16_to_f64(h)
        assert oracle.f32_to_f16(v) == h, hex(h)


def test_f16_decode_known():
    assert oracle.f16_to_f64(0x3C00) == 1.0
    assert oracle.f16_to_f64(0x0001) == 2.0 ** -24
    assert oracle.f16_to_f64(0x7BFF) == 65504.0
    assert oracle.f16_to_f64(0xBC00) == -1.0


def test_quant_properties_random():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((4, 4096)) * rng.uniform(1e-3, 1e3, (4, 1))).astype(np.float32)
    qs, d16 = oracle.quant_q8(x)
    xb = x.reshape(-1, 32)
    qb = qs.reshape(-1, 32).astype(np.int32)
    amax = np.abs(xb).max(axis=1)
    d = (amax / np.float32(127)).astype(np.float32)
    di = (np.float32(1) / d).astype(np.float32)
    prod = (xb * di[:, None]).astype(np.float32)
    # every code is the nearest integer to the f32 product (no clamp reached)
    assert np.all(np.abs(prod - qb) <= 0.5)
    # the largest-magnitude element maps to +-127 (or +-126 through rounding of di)
    top = qb[np.arange(len(qb)), np.abs(xb).argmax(axis=1)]
    assert np.all(np.abs(top) >= 126) and np.all(np.abs(qb) <= 127)
    assert np.array_equal(d16.reshape(-1), d.astype(np.float16).view(np.uint16))


def test_quant_power_of_two_scaling():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 1024)).astype(np.float32)
    q1, d1 = oracle.quant_q8(x)
    q2, d2 = oracle.quant_q8(x * np.float32(4.0))
    assert np.array_equal(q1, q2)
    assert np.array_equal(d2.astype(np.int32), d1.astype(np.int32) + (2 << 10))


def test_quant_rejects_nonfinite():
    x = np.zeros((1, 32), np.float32)
    x[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.quant_q8(x)


def test_rmsnorm_constant_row():
    # mean(x^2) = 4 -> r = 1/2 exactly (eps = 0): y = (2 * 0.5) * gamma = gamma
    K = 64
    g = np.linspace(0.5, 1.5, K).astype(np.float32)
    y = oracle.rmsnorm(np.full((1, K), 2.0, np.float32), g, 0.0)
    assert np.array_equal(y[0], g)


def test_rmsnorm_pythagorean_row():
    # x = [3, 4, 0, 0]: mean(x^2) = 25/4, r = 1/2.5 = 0.4 (rounded to f32)
    x = np.array([[3, 4, 0, 0]], np.float32)
    g = np.array([1, 1, 1, 1], np.float32)
    y = oracle.rmsnorm(x, g, 0.0)
    r = np.float32(0.4)
    assert np.array_equal(y[0], np.array([np.float32(3) * r, np.float32(4) * r, 0, 0], np.float32))


def test_rmsnorm_zero_row_and_scaling():
    K = 256
    g = np.ones(K, np.float32)
    assert not oracle.rmsnorm(np.zeros((1, K), np.float32), g, 1e-6).any()
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, K)).astype(np.float32)
    y1 = oracle.rmsnorm(x, g, 0.0)
    y2 = oracle.rmsnorm(x * np.float32(8.0), g, 0.0)
    assert np.array_equal(y1, y2)
    # rows are normalised independently; unit gamma gives mean(y^2) = 1
    assert np.allclose((y1.astype(np.float64) ** 2).mean(axis=1), 1.0, rtol=1e-6)


def test_rmsnorm_eps_enters_inside_the_root():
    # x = 1 everywhere: r = 1/sqrt(1 + eps)
    K = 32
    y = oracle.rmsnorm(np.ones((1, K), np.float32), np.ones(K, np.float32), 0.25)
    assert np.all(y == np.float32(1 / np.sqrt(1.25)))


# --- SwiGLU (silu(g) * u) --------------------------------------------------------

def test_swiglu_textbook_values():
    # silu(0) = 0; silu(1) = 1/(1 + e^-1) = 0.7310585786300049 (sigma(1)); silu(-1) =
    # -0.2689414213699951; at g = +-40 the logistic saturates: silu(40) = 40 in f32 and
    # silu(-40) = -40 e^-40 / (1 + e^-40) = -1.6993e-16.
    g = np.array([[0.0, 1.0, -1.0, 40.0, -40.0, 2.0]], np.float32)
    u = np.ones_like(g)
    y = oracle.swiglu(g, u)[0]
    assert y[0] == 0.0
    assert y[1] == np.float32(0.7310585786300049)
    assert y[2] == np.float32(-0.2689414213699951)
    assert y[3] == np.float32(40.0)
    assert abs(y[4] - np.float32(-1.6993417021166355e-16)) <= np.spacing(np.float32(1.7e-16))
    assert y[5] == np.float32(1.7615941559557649)   # 2 * sigma(2)


def test_swiglu_odd_part_identity():
    # silu(x) - silu(-x) = x exactly in real arithmetic; with one f32 rounding of each
    # term the difference is within an ulp of each.
    rng = np.random.default_rng(21)
    g = rng.standard_normal((1, 4096)).astype(np.float32) * np.float32(4)
    one = np.ones_like(g)
    a = oracle.swiglu(g, one).astype(np.float64)
    b = oracle.swiglu(-g, one).astype(np.float64)
    tol = np.spacing(np.abs(a).astype(np.float32)) + np.spacing(np.abs(b).astype(np.float32))
    assert np.all(np.abs((a - b) - g.astype(np.float64)) <= tol)


def test_swiglu_is_linear_in_u_and_zero_rows():
    rng = np.random.default_rng(22)
    g = rng.standard_normal((2, 512)).astype(np.float32)
    u = rng.standard_normal((2, 512)).astype(np.float32)
    y1 = oracle.swiglu(g, u)
    y2 = oracle.swiglu(g, u * np.float32(4))          # power-of-two scaling is exact
    assert np.array_equal(y2, y1 * np.float32(4))
    assert not oracle.swiglu(g, np.zeros_like(u)).any()
    assert not oracle.swiglu(np.zeros_like(g), u).any()
