"""GPU parity of the q4_K / q5_K split-plane GEMV against the oracle: device repack
byte for byte, exact code dots, the GEMV on full-size workloads and dispatch edges,
exact coverage sums, the one-hot probe, and the fused RMSNorm -> q8 -> GEMV call."""
import numpy as np
import pytest
import torch

import oracle
import q6ksynth
import quantized_decode_gemv_amd as q
from gpu_util import (DEV, check_plane_vs_oracle_chain, check_y, check_y_on_plane, dev_f32,
                      dev_u8, make_plane, oracle_threads, q8_plane, say, split_plane)
from kq_build import blank, set_code, set_d, set_scale_min

pytestmark = pytest.mark.gpu

TYPES = [q.KQ_Q4_K, q.KQ_Q5_K]
NAMES = {q.KQ_Q4_K: "q4_K", q.KQ_Q5_K: "q5_K"}


def _ids(t):
    return NAMES[t]


def kq_dpl_from_raw(qtype, raw, N, K):
    raw_d = dev_u8(raw)
    assert raw_d.numel() == q.kq_raw_bytes(qtype, N, K)
    dpl = torch.empty(q.kq_dpl_bytes(qtype, N, K), dtype=torch.uint8, device=DEV)
    q.repack_kq_dpl(qtype, raw_d, dpl, N, K)
    return dpl


def run_kq(qtype, dpl, plane, N, K, nt):
    y = torch.full((nt, N), float("nan"), dtype=torch.float32, device=DEV)
    q.mmvq_kq_q8(qtype, dpl, plane, y, N, K, nt)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("N,K", [(1, 256), (7, 5120), (3, 256 * 97), (27648, 5120)])
def test_device_repack_byte_exact(qtype, N, K):
    raw = q6ksynth.raw_kq(qtype, N, K, seed=N + K)
    dpl = torch.full((q.kq_dpl_bytes(qtype, N, K),), 0xEE, dtype=torch.uint8, device=DEV)
    q.repack_kq_dpl(qtype, dev_u8(raw), dpl, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(dpl.cpu().numpy(), oracle.kq_repack_dpl(qtype, raw, N, K))


# The raw matrix may start at any address: word reads where its base allows them,
# byte reads otherwise (q6_K: 16-bit reads on an even base).
@pytest.mark.parametrize("qtype", [q.KQ_Q4_K, q.KQ_Q5_K, q.KQ_Q6_K])
@pytest.mark.parametrize("shift", [0, 1, 2, 3])
def test_device_repack_any_raw_alignment(qtype, shift):
    N, K = 5, 256 * 7
    raw = (q6ksynth.raw_q6k(N, K, seed=9 + shift) if qtype == q.KQ_Q6_K
           else q6ksynth.raw_kq(qtype, N, K, seed=9 + shift))
    flat = torch.from_numpy(raw.reshape(-1)).to(DEV)
    buf = torch.zeros(flat.numel() + 16, dtype=torch.uint8, device=DEV)
    buf[shift:shift + flat.numel()] = flat
    dpl = torch.full((q.kq_dpl_bytes(qtype, N, K),), 0xEE, dtype=torch.uint8, device=DEV)
    q.repack_kq_dpl(qtype, buf[shift:shift + flat.numel()], dpl, N, K)
    torch.cuda.synchronize()
    expect = (oracle.repack_dpl(raw, N, K) if qtype == q.KQ_Q6_K
              else oracle.kq_repack_dpl(qtype, raw, N, K))
    assert np.array_equal(dpl.cpu().numpy(), expect)


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("N,K,nt", [(64, 1024, 1), (37, 5120, 2), (5, 13824, 3),
                                    (3, 256 * 97, 1), (2, 256 * 200, 5)])
def test_subdots_bit_exact(qtype, N, K, nt):
    raw = q6ksynth.raw_kq(qtype, N, K, seed=N * 7 + nt + qtype)
    dpl = kq_dpl_from_raw(qtype, raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 950 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    dots = torch.zeros((nt, N, K // 32), dtype=torch.int32, device=DEV)
    q.mmvq_kq_q8_subdots(qtype, dpl, make_plane(qs, d), dots, N, K, nt)
    torch.cuda.synchronize()
    assert np.array_equal(dots.cpu().numpy(), oracle.kq_subdots(qtype, oracle.RAW, raw, N, K, qs))


@pytest.mark.parametrize("name,nt", [("q4k_gate_up", 1), ("q4k_gate_up", 4), ("q4k_down", 1),
                                     ("q5k_gate_up", 1), ("q5k_gate_up", 4), ("q5k_down", 1)])
def test_workload_full_parity(name, nt):
    """Every output at full size, on the oracle's q8 plane."""
    w = q6ksynth.WORKLOADS[name]
    say(f"workload {name} N={w.N} K={w.K} nt={nt}")
    raw = q6ksynth.weights(w)
    dpl = kq_dpl_from_raw(w.qtype, raw, w.N, w.K)
    if w.producer == "swiglu":
        g, u = q6ksynth.swiglu_pairs(w, nt)
        x = oracle.swiglu(g, u)
    else:
        x = oracle.rmsnorm(q6ksynth.activations(w, nt), q6ksynth.gamma(w.K, q6ksynth.gamma_seed(w)),
                           q6ksynth.RMS_EPS)
    qs, d = oracle.quant_q8(x)
    y = run_kq(w.qtype, dpl, make_plane(qs, d), w.N, w.K, nt)
    y_or, A = oracle.kq_mmvq(w.qtype, oracle.RAW, raw, w.N, w.K, qs, d, nthreads=oracle_threads())
    worst = check_y(y, y_or, A, name)
    say(f"  max err/A = {worst:.3e}")


EDGE_NBE = sorted({1, 2, 3, 7, 8, 9, 16, 17, 24, 25, 48, 49, 56, 57, 96, 97, 128, 200})


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("nbe", EDGE_NBE)
@pytest.mark.parametrize("nt", [1, 2, 4, 5])
def test_dispatch_edges_random(qtype, nbe, nt):
    K, N = 256 * nbe, 67
    raw = q6ksynth.raw_kq(qtype, N, K, seed=nbe * 10 + nt + qtype)
    dpl = kq_dpl_from_raw(qtype, raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 1100 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_kq(qtype, dpl, make_plane(qs, d), N, K, nt)
    y_or, A = oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, qs, d)
    check_y(y, y_or, A, f"{NAMES[qtype]} nbe={nbe} nt={nt}")


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("N,nbe,nt", [(2999, 54, 1), (2999, 74, 4), (1237, 96, 2),
                                      (2001, 48, 3)])
def test_shared_rows_random(qtype, N, nbe, nt):
    # rows shared by the workgroup's four waves: several per workgroup, a short last one
    K = 256 * nbe
    p = q.mmvq_plan(N, K, nt, 256, qtype)
    assert p["shared"]
    raw = q6ksynth.raw_kq(qtype, N, K, seed=N + nbe * 10 + nt + qtype)
    dpl = kq_dpl_from_raw(qtype, raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 1300 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_kq(qtype, dpl, make_plane(qs, d), N, K, nt)
    y_or, A = oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, qs, d, nthreads=oracle_threads())
    check_y(y, y_or, A, f"{NAMES[qtype]} shared N={N} nbe={nbe} nt={nt}")


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("nbe", [4, 12, 20])
@pytest.mark.parametrize("N,nt", [(4095, 2), (4097, 4), (6001, 3)])
def test_pairs_random(qtype, nbe, N, nt):
    # two rows per wave, the last chunk slot split between them
    K = 256 * nbe
    assert q.mmvq_plan(N, K, nt, 256, qtype)["paired"]
    raw = q6ksynth.raw_kq(qtype, N, K, seed=N * 3 + nbe + nt + qtype)
    dpl = kq_dpl_from_raw(qtype, raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 1500 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_kq(qtype, dpl, make_plane(qs, d), N, K, nt)
    y_or, A = oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, qs, d)
    check_y(y, y_or, A, f"{NAMES[qtype]} pairs N={N} nbe={nbe} nt={nt}")


# q4_K / q5_K matrices past 4 GiB of split-plane rows (K = 5120; 1.5M q4_K rows, 1.3M
# q5_K rows): rows past byte 2^32 need wider offsets in the repack and the GEMV. Raw
# blocks are made on the device from a seeded generator (uniform bytes, d and dmin =
# fp16(|N(0,1)| * 1e-3)); the oracle checks the first and last rows and a sample.
@pytest.mark.parametrize("qtype,N,nt", [(q.KQ_Q4_K, 1500000, 1), (q.KQ_Q5_K, 1300000, 2)],
                         ids=["q4_K-1", "q5_K-2"])
def test_matrix_past_4gib(qtype, N, nt):
    K = 5120
    nbe, B = K // 256, q.kq_block_bytes(qtype)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4343 + qtype)
    raw = torch.randint(0, 256, (N, nbe, B), dtype=torch.uint8, device=DEV, generator=gen)
    dm = (torch.randn((N, nbe, 2), device=DEV, generator=gen).abs() * 1e-3).half()
    raw[:, :, 0:4] = dm.view(torch.uint8).view(N, nbe, 4)
    dpl = torch.empty(q.kq_dpl_bytes(qtype, N, K), dtype=torch.uint8, device=DEV)
    q.repack_kq_dpl(qtype, raw.view(-1), dpl, N, K)
    assert dpl.numel() > (1 << 32)
    x = np.stack([q6ksynth.activation("outlier", K, 1700 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_kq(qtype, dpl, make_plane(qs, d), N, K, nt)
    del dpl
    rng = np.random.default_rng(4344 + qtype)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(N - 512, N),
                                     rng.integers(0, N, 512)]))
    raw_h = raw[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del raw
    torch.cuda.empty_cache()
    y_or, A = oracle.kq_mmvq(qtype, oracle.RAW, raw_h.reshape(-1), rows.size, K, qs, d,
                             nthreads=oracle_threads())
    worst = check_y(y[:, rows], y_or, A, f"{NAMES[qtype]} past 4 GiB N={N} nt={nt}")
    say(f"{NAMES[qtype]} past 4 GiB N={N} nt={nt}: {rows.size} rows, max err/A = {worst:.3e}")


def _uniform_block(qtype, code, sc, m, d, dmin):
    blk = blank(qtype, 1)[0]
    set_d(qtype, blk, d, dmin)
    for s in range(8):
        set_scale_min(qtype, blk, s, sc, m)
    for e in range(256):
        set_code(qtype, blk, e, code)
    return blk


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("nbe", [1, 2, 7, 8, 9, 20, 54, 74, 96, 97, 128])
@pytest.mark.parametrize("N", [1, 3, 64, 65, 257, 4097])
def test_coverage_exact_sum(qtype, nbe, N):
    """Codes all c, scale 1, min 1, d = dmin = 1, activations all 1 (d8 = 1):
    y = (c - 1) * K exactly. A dropped unit or a counted-twice one shows as an exact
    difference."""
    K = 256 * nbe
    c = 3 if qtype == q.KQ_Q4_K else 19
    blk = _uniform_block(qtype, c, 1, 1, 1.0, 1.0)
    raw = np.tile(blk, (N, nbe))
    dpl = kq_dpl_from_raw(qtype, raw, N, K)
    for nt in (1, 2, 5):
        qs = np.ones((nt, K), np.int8)
        d = np.full((nt, K // 32), np.float16(1.0).view(np.uint16), np.uint16)
        y = run_kq(qtype, dpl, make_plane(qs, d), N, K, nt)
        assert np.all(y == (c - 1) * K), (nt, np.unique(y)[:5])


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("q0", [1, 9, 15, 17, 31])
def test_onehot_diagonal(qtype, q0):
    if qtype == q.KQ_Q4_K and q0 > 15:
        pytest.skip("q4_K codes are 4 bits")
    raw = blank(qtype, 256)
    for e in range(256):
        set_d(qtype, raw[e], 1.0, 1.0)
        for s in range(8):
            set_scale_min(qtype, raw[e], s, s + 1, 0)
        set_code(qtype, raw[e], e, q0)
    qs = np.eye(256, dtype=np.int8)
    d16 = np.full((256, 8), np.float16(1.0).view(np.uint16), np.uint16)
    y = run_kq(qtype, kq_dpl_from_raw(qtype, raw, 256, 256), make_plane(qs, d16), 256, 256, 256)
    expect = np.diag([(e // 32 + 1) * q0 for e in range(256)]).astype(np.float32)
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("name,nt", [("q4k_gate_up", 1), ("q5k_gate_up", 1), ("q4k_gate_up", 4)])
def test_fused_rmsnorm_equals_two_kernels(name, nt):
    w = q6ksynth.WORKLOADS[name]
    assert q.rmsnorm_mmvq_fused(w.N, w.K, nt) == (nt == 1)
    raw = q6ksynth.weights(w)
    dpl = kq_dpl_from_raw(w.qtype, raw, w.N, w.K)
    x = q6ksynth.activations(w, nt)
    g = q6ksynth.gamma(w.K, q6ksynth.gamma_seed(w))
    xd, gd = dev_f32(x), dev_f32(g)
    p1, p2 = q8_plane(w.K, nt), q8_plane(w.K, nt)
    y1 = torch.empty((nt, w.N), dtype=torch.float32, device=DEV)
    y2 = torch.empty_like(y1)
    xn = torch.empty((nt, w.K), dtype=torch.float32, device=DEV)
    q.mmvq_kq_rmsnorm_q8(w.qtype, dpl, xd, gd, q6ksynth.RMS_EPS, None, p1, y1, w.N, w.K, nt)
    q.rmsnorm_quant_q8(xd, gd, q6ksynth.RMS_EPS, xn, p2, w.K, nt)
    q.mmvq_kq_q8(w.qtype, dpl, p2, y2, w.N, w.K, nt)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    # and against the oracle chain where the q8 planes agree
    x_or = oracle.rmsnorm(x, g, q6ksynth.RMS_EPS)
    qs_or, d_or = oracle.quant_q8(x_or)
    qs, d = split_plane(p1, w.K, nt)
    rep = check_plane_vs_oracle_chain(xn.cpu().numpy(), x_or, qs, d, qs_or, d_or, name)
    # y against the oracle GEMV on the fused kernel's own q8 plane, always
    rep["max_err_over_A"] = check_y_on_plane(y1.cpu().numpy(), raw, qs, d, w.N, w.K,
                                             name + " fused", qtype=w.qtype)
    say(f"{name} nt={nt}: fused == producer + GEMV bitwise; {rep}")
