"""GPU parity: device repack and the q8 producers against the oracle (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
import q6ksynth
import quantized_decode_gemv_amd as q
from golden_io import q8_cases
from gpu_util import (DEV, check_plane_vs_oracle_chain, dev_f32, dev_u8, dpl_from_raw, q8_plane,
                      say, split_plane, swiglu_tol)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(1, 256), (3, 1024), (64, 1024), (7, 13824), (5, 18944),
                                 (33, 256 * 97), (1024, 5120)])
def test_device_repack_is_byte_exact(N, K):
    say(f"repack N={N} K={K}")
    raw = q6ksynth.raw_q6k(N, K, seed=100 + N)
    dpl = dpl_from_raw(raw, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(dpl.cpu().numpy(), oracle.repack_dpl(raw, N, K))


def test_device_repack_full_lm_head_shape():
    w = q6ksynth.WORKLOADS["lm_head"]
    say("repack lm_head full shape")
    raw = q6ksynth.weights(w)
    dpl = dpl_from_raw(raw, w.N, w.K)
    torch.cuda.synchronize()
    assert np.array_equal(dpl.cpu().numpy(), oracle.repack_dpl(raw, w.N, w.K))


def test_device_repack_overwrites_pad_bytes():
    N, K = 5, 1024
    raw = q6ksynth.raw_q6k(N, K, seed=3)
    dpl = torch.full((q.q6k_dpl_bytes(N, K),), 0xEE, dtype=torch.uint8, device=DEV)
    q.repack_q6k_dpl(dev_u8(raw), dpl, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(dpl.cpu().numpy(), oracle.repack_dpl(raw, N, K))


@pytest.mark.parametrize("case", q8_cases(), ids=lambda c: c[0])
def test_quant_q8_closed_form(case):
    _, x, qexp, d16 = case
    plane = q8_plane(32, 1)
    q.quant_q8(dev_f32(x), plane, 32, 1)
    qs, d = split_plane(plane, 32, 1)
    assert np.array_equal(qs[0], qexp) and int(d[0, 0]) == d16


@pytest.mark.parametrize("K", [32, 256, 1024, 5120, 13824, 18944, 1 << 20])
@pytest.mark.parametrize("nt", [1, 4, 5])
@pytest.mark.parametrize("kind", ["normal", "outlier", "swiglu"])
def test_quant_q8_bit_exact(K, nt, kind):
    if kind == "swiglu":   # SwiGLU-shaped rows (the oracle's silu(g) * u)
        x = np.stack([oracle.swiglu(*q6ksynth.swiglu_pair(K, 500 + c))[0] for c in range(nt)])
    else:
        x = np.stack([q6ksynth.activation(kind, K, 500 + c) for c in range(nt)])
    plane = q8_plane(K, nt)
    q.quant_q8(dev_f32(x), plane, K, nt)
    qs, d = split_plane(plane, K, nt)
    qs_o, d_o = oracle.quant_q8(x)
    assert np.array_equal(qs, qs_o) and np.array_equal(d, d_o)


def test_quant_q8_wide_dynamic_range():
    rng = np.random.default_rng(4)
    K, nt = 8192, 3
    scale = np.float32(10.0) ** rng.integers(-6, 6, size=(nt, K // 32, 1)).astype(np.float32)
    x = (rng.standard_normal((nt, K // 32, 32)).astype(np.float32) * scale).reshape(nt, K)
    x[0, :32] = 0.0
    plane = q8_plane(K, nt)
    q.quant_q8(dev_f32(x), plane, K, nt)
    qs, d = split_plane(plane, K, nt)
    qs_o, d_o = oracle.quant_q8(x)
    assert np.array_equal(qs, qs_o) and np.array_equal(d, d_o)


# every register-resident variant's edge (K/4 = 512, 1024, 2048, 4096, 8192 float4s)
# and the looping form past K = 32768
# up to the longest row the boundary accepts (K = 2^20)
RMS_K = [256, 1024, 2048, 2080, 4096, 4128, 5120, 8192, 8224, 13824, 16384, 16416, 18944,
         32768, 32800, 40960, 1 << 20]


@pytest.mark.parametrize("K", RMS_K)
@pytest.mark.parametrize("nt", [1, 4])
def test_rmsnorm_quant_q8(K, nt):
    """y within the reading's tolerance (the reduction order is free); the q8 plane
    against the oracle chain, block by block (check_plane_vs_oracle_chain)."""
    x = np.stack([q6ksynth.activation("outlier", K, 700 + c) for c in range(nt)])
    g = q6ksynth.gamma(K, 701)
    y = torch.empty((nt, K), dtype=torch.float32, device=DEV)
    plane = q8_plane(K, nt)
    q.rmsnorm_quant_q8(dev_f32(x), dev_f32(g), q6ksynth.RMS_EPS, y, plane, K, nt)
    y_gpu = y.cpu().numpy()
    y_or = oracle.rmsnorm(x, g, q6ksynth.RMS_EPS)
    ulp = np.spacing(np.abs(y_or))
    assert np.all(np.abs(y_gpu - y_or) <= 2 * ulp)
    qs, d = split_plane(plane, K, nt)
    qs_or, d_or = oracle.quant_q8(y_or)
    rep = check_plane_vs_oracle_chain(y_gpu, y_or, qs, d, qs_or, d_or, f"K={K} nt={nt}")
    say(f"rmsnorm K={K} nt={nt}: y bit-equal fraction {np.mean(y_gpu == y_or):.6f}; {rep}")


def test_rmsnorm_zero_row_is_zero():
    K = 1024
    x = np.zeros((1, K), np.float32)
    y = torch.empty((1, K), dtype=torch.float32, device=DEV)
    plane = q8_plane(K, 1)
    q.rmsnorm_quant_q8(dev_f32(x), dev_f32(np.ones(K, np.float32)), 1e-6, y, plane, K, 1)
    assert not y.cpu().numpy().any()
    qs, d = split_plane(plane, K, 1)
    assert not qs.any() and not d.any()


# --- fused SwiGLU -> q8 -------------------------------------------------------------

@pytest.mark.parametrize("K", [32, 256, 5120, 13824, 18944, 1 << 20])
@pytest.mark.parametrize("nt", [1, 4, 5])
def test_swiglu_quant_q8(K, nt):
    g, u = (np.stack(a) for a in zip(*[q6ksynth.swiglu_pair(K, 800 + c) for c in range(nt)]))
    # saturation, zeros, and gates past the f32 overflow of expf(-g) (g < -88.7)
    g[0, :12] = [0.0, 40.0, -40.0, 88.0, -88.0, 1e-30, -3.0, 3.0, -89.0, -95.0, -103.0, -200.0]
    y = torch.empty((nt, K), dtype=torch.float32, device=DEV)
    plane = q8_plane(K, nt)
    q.swiglu_quant_q8(dev_f32(g), dev_f32(u), y, plane, K, nt)
    y_gpu = y.cpu().numpy()
    y_or = oracle.swiglu(g, u)
    assert np.all(np.abs(y_gpu.astype(np.float64) - y_or) <= swiglu_tol(y_or, g, u))
    qs, d = split_plane(plane, K, nt)
    qs_or, d_or = oracle.quant_q8(y_or)
    rep = check_plane_vs_oracle_chain(y_gpu, y_or, qs, d, qs_or, d_or, f"swiglu K={K} nt={nt}")
    say(f"swiglu K={K} nt={nt}: y bit-equal fraction {np.mean(y_gpu == y_or):.4f}; {rep}")


@pytest.mark.parametrize("which", ["g", "u"])
def test_swiglu_in_place(which):
    K, nt = 5120, 2
    g, u = (np.stack(a) for a in zip(*[q6ksynth.swiglu_pair(K, 810 + c) for c in range(nt)]))
    gd, ud = dev_f32(g), dev_f32(u)
    ref = torch.empty((nt, K), dtype=torch.float32, device=DEV)
    p_ref = q8_plane(K, nt)
    q.swiglu_quant_q8(gd, ud, ref, p_ref, K, nt)
    p_in = q8_plane(K, nt)
    out = gd if which == "g" else ud
    q.swiglu_quant_q8(gd, ud, out, p_in, K, nt)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(p_in, p_ref)
