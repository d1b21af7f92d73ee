"""GPU parity: exact sub-block dots and the GEMV against the oracle, on every
workload (full size, every output compared) plus dispatch edges."""
import numpy as np
import pytest
import torch

import oracle
import q6ksynth
import quantized_decode_gemv_amd as q
from gpu_util import (DEV, check_plane_vs_oracle_chain, check_y, check_y_on_plane, dev_f32,
                      dpl_from_raw, make_plane, oracle_threads, q8_plane, run_mmvq, say,
                      split_plane)
from q6k_build import onehot_probe

pytestmark = pytest.mark.gpu


def _chain(w: q6ksynth.Workload, nt: int):
    """The workload's whole path on the GPU (device repack, its producer, the GEMV)
    and on the oracle (repack-free raw rows, producer, GEMV), from the same seeds."""
    raw = q6ksynth.weights(w)
    dpl = dpl_from_raw(raw, w.N, w.K)
    plane = q8_plane(w.K, nt)
    if w.producer != "swiglu":
        x = q6ksynth.activations(w, nt)
    if w.producer == "rmsnorm":
        g = q6ksynth.gamma(w.K, q6ksynth.gamma_seed(w))
        yd = torch.empty((nt, w.K), dtype=torch.float32, device=DEV)
        q.rmsnorm_quant_q8(dev_f32(x), dev_f32(g), q6ksynth.RMS_EPS, yd, plane, w.K, nt)
        x_or = oracle.rmsnorm(x, g, q6ksynth.RMS_EPS)
        x_gpu = yd.cpu().numpy()
    elif w.producer == "swiglu":
        gate, up = q6ksynth.swiglu_pairs(w, nt)
        yd = torch.empty((nt, w.K), dtype=torch.float32, device=DEV)
        q.swiglu_quant_q8(dev_f32(gate), dev_f32(up), yd, plane, w.K, nt)
        x_or = oracle.swiglu(gate, up)
        x_gpu = yd.cpu().numpy()
    else:
        q.quant_q8(dev_f32(x), plane, w.K, nt)
        x_or = x_gpu = x
    qs_or, d_or = oracle.quant_q8(x_or)
    return raw, dpl, plane, x_gpu, x_or, qs_or, d_or


@pytest.mark.parametrize("name,nt", [("tiny", 1), ("attn_v", 1), ("ffn_down", 1), ("tall_k", 1),
                                     ("lm_head", 1), ("lm_head", 4)])
def test_workload_full_parity(name, nt):
    """Every output of every workload at full size. The GEMV is checked on the
    oracle's q8 plane (both sides consume identical inputs). The GPU's own chain
    (producer -> GEMV) is checked too: its q8 plane bit for bit against the oracle
    quantizer of the producer's own y, and its y against the oracle GEMV on that
    plane; where that plane equals the oracle chain's, the two GPU runs must agree
    bit for bit."""
    w = q6ksynth.WORKLOADS[name]
    say(f"workload {name} N={w.N} K={w.K} nt={nt}")
    raw, dpl, plane, x_gpu, x_or, qs_or, d_or = _chain(w, nt)
    y_or, A = oracle.mmvq(oracle.RAW, raw, w.N, w.K, qs_or, d_or, nthreads=oracle_threads())
    y = run_mmvq(dpl, make_plane(qs_or, d_or), w.N, w.K, nt)
    worst = check_y(y, y_or, A, name)
    say(f"  GEMV on the oracle's q8: max err/A = {worst:.3e}")
    qs, d = split_plane(plane, w.K, nt)
    rep = check_plane_vs_oracle_chain(x_gpu, x_or, qs, d, qs_or, d_or, name)
    say(f"  producer plane vs oracle chain: {rep}")
    y_chain = run_mmvq(dpl, plane, w.N, w.K, nt)
    worst_chain = check_y_on_plane(y_chain, raw, qs, d, w.N, w.K, name + " chain")
    say(f"  GPU chain vs the oracle GEMV on the GPU's plane: max err/A = {worst_chain:.3e}")
    if rep["codes_differ"] == 0 and np.array_equal(d, d_or):
        assert np.array_equal(y_chain, y)
    if name == "lm_head":
        for t in range(nt):
            top = np.argsort(y_or[t])[-2:]
            margin = y_or[t, top[1]] - y_or[t, top[0]]
            g = int(np.argmax(y[t]))
            ok = g == top[1] or (margin <= 2 * 1e-5 * A[t, top].max() and g == top[0])
            say(f"  token {t}: argmax gpu {g} oracle {top[1]} margin {margin:.4g}")
            assert ok


@pytest.mark.parametrize("N,K,nt", [(64, 1024, 1), (1024, 5120, 1), (37, 13824, 2),
                                    (5, 18944, 3), (3, 256 * 97, 1), (2, 256 * 200, 5)])
def test_subdots_bit_exact(N, K, nt):
    say(f"subdots N={N} K={K} nt={nt}")
    raw = q6ksynth.raw_q6k(N, K, seed=N * 7 + nt)
    dpl = dpl_from_raw(raw, N, K)
    x = np.stack([oracle.swiglu(*q6ksynth.swiglu_pair(K, 900 + c))[0] for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    plane = make_plane(qs, d)
    dots = torch.zeros((nt, N, K // 16), dtype=torch.int32, device=DEV)
    q.mmvq_q6k_q8_subdots(dpl, plane, dots, N, K, nt)
    torch.cuda.synchronize()
    assert np.array_equal(dots.cpu().numpy(), oracle.subdots(oracle.RAW, raw, N, K, qs))


# chunks per lane change at nbe = 8k -> 8k+1; the unrolled/generic switch is at
# nbe 96 -> 97; the operand mode (registers or LDS), the shared rows (from 7 chunks
# per lane) and the row pairs (nbe 4, 12, 20 at several tokens, enough rows) switch
# with chunks per lane and tokens.
EDGE_NBE = sorted({1, 2, 3, 7} | {8 * k for k in range(1, 13)} | {8 * k + 1 for k in range(0, 13)}
                  | {100, 128, 200})


@pytest.mark.parametrize("nbe", EDGE_NBE)
@pytest.mark.parametrize("nt", [1, 2, 3, 4, 5])
def test_dispatch_edges_random(nbe, nt):
    K, N = 256 * nbe, 67
    raw = q6ksynth.raw_q6k(N, K, seed=nbe * 10 + nt)
    dpl = dpl_from_raw(raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 1000 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_mmvq(dpl, make_plane(qs, d), N, K, nt)
    y_or, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d)
    check_y(y, y_or, A, f"nbe={nbe} nt={nt}")


# Long rows that the workgroup's four waves share (chunks per lane 7..12, or 6 from 3
# tokens): several rows per workgroup, a short last workgroup (N not a multiple of
# the rows per workgroup), both of its chunk counts per thread (2: nbe 49..64, 3:
# nbe 65..96), one token (q6_K shares them when the rows are few) and several.
@pytest.mark.parametrize("N,nbe,nt", [(2999, 54, 1), (2999, 54, 2), (2999, 74, 1),
                                      (2999, 74, 4), (1237, 96, 3), (4097, 49, 5),
                                      (2001, 48, 3), (3584, 74, 4)])
def test_shared_rows_random(N, nbe, nt):
    K = 256 * nbe
    p = q.mmvq_plan(N, K, nt, 256)
    say(f"shared rows N={N} nbe={nbe} nt={nt}: plan {p}")
    assert p["shared"]
    raw = q6ksynth.raw_q6k(N, K, seed=N + nbe * 10 + nt)
    dpl = dpl_from_raw(raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 1200 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_mmvq(dpl, make_plane(qs, d), N, K, nt)
    y_or, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d, nthreads=oracle_threads())
    check_y(y, y_or, A, f"N={N} nbe={nbe} nt={nt}")


# Two rows per wave (2..4 tokens, rows of an odd multiple of 32 chunks: nbe 4, 12, 20):
# every chunk count per lane 1..3, an odd N (the last pair has one row), and nt = 5 (a
# paired launch of 4 tokens, then a one-wave launch of 1). With many more rows, rows of 20
# super-blocks at 3 and 4 tokens take the matrix-core tiles instead (test_tiles_random).
@pytest.mark.parametrize("nbe", [4, 12, 20])
@pytest.mark.parametrize("N,nt", [(4095, 2), (4097, 3), (8192, 4), (4099, 5), (4095, 4),
                                  (4097, 4)])
def test_pairs_random(nbe, N, nt):
    K = 256 * nbe
    plan = q.mmvq_plan(N, K, nt, 256)
    assert plan["paired"] and not plan["tiles"]
    raw = q6ksynth.raw_q6k(N, K, seed=N * 3 + nbe + nt)
    dpl = dpl_from_raw(raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 1400 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_mmvq(dpl, make_plane(qs, d), N, K, nt)
    y_or, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d)
    check_y(y, y_or, A, f"pairs N={N} nbe={nbe} nt={nt}")


# 16-row tiles on the int8 matrix cores (q6_K, K = 5120; 4 tokens per launch from 12 tiles
# per CU, 3 from 24): the first row count that takes them at 4 and at 3 tokens (whole
# rounds of tiles), a ragged last tile (N % 16 = 1 and 15) with a partial last round, 5
# and 7 tokens (a tile launch of 4, then 1 or 3 more), and a zero activation row next to
# nonzero ones (its outputs must be exactly 0).
TILES_4 = 16 * 12 * 256
TILES_3 = 16 * 24 * 256


@pytest.mark.parametrize("N,nt", [(TILES_4, 4), (TILES_4 + 1, 4), (TILES_3, 3), (TILES_3 + 15, 3),
                                  (TILES_4 + 4111, 4), (TILES_4 + 333, 5), (TILES_4 + 17, 7)])
def test_tiles_random(N, nt):
    K = 5120
    plan = q.mmvq_plan(N, K, nt, 256)
    assert plan["tiles"] and plan["grid"] == min(-(-N // 16), 256)
    say(f"tiles N={N} nt={nt}")
    raw = q6ksynth.raw_q6k(N, K, seed=N * 5 + nt)
    dpl = dpl_from_raw(raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 1600 + c) for c in range(nt)])
    x[1] = 0.0
    qs, d = oracle.quant_q8(x)
    y = run_mmvq(dpl, make_plane(qs, d), N, K, nt)
    y_or, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d, nthreads=oracle_threads())
    assert np.all(y[1] == 0)
    check_y(y, y_or, A, f"tiles N={N} nt={nt}")


# Matrices past 4 GiB of dpl rows: the rows past byte 2^32 need wider than 32-bit
# offsets, in the repack and in the GEMV kinds that reach such sizes -- lm_head-width
# rows (2^20 of them) at one token (one wave per row) and four (matrix-core tiles); tall-K
# rows at four tokens (operands staged in LDS); rows of 100 super-blocks (the generic
# stepping kernel). The raw blocks are made on the device from a seeded generator
# (uniform bytes, d = fp16(|N(0,1)| * 1e-3)); the oracle checks the first and last
# rows and a seeded sample between them.
@pytest.mark.parametrize("N,K,nt", [(1 << 20, 5120, 1), (1 << 20, 5120, 4),
                                    (280000, 18944, 4), (210000, 25600, 1)])
def test_matrix_past_4gib(N, K, nt):
    nbe = K // 256
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4242)
    raw = torch.randint(0, 256, (N, nbe, 210), dtype=torch.uint8, device=DEV, generator=gen)
    d = (torch.randn((N, nbe), device=DEV, generator=gen).abs() * 1e-3).half()
    raw[:, :, 208:210] = d.view(torch.uint8).view(N, nbe, 2)
    dpl = torch.empty(q.q6k_dpl_bytes(N, K), dtype=torch.uint8, device=DEV)
    q.repack_q6k_dpl(raw.view(-1), dpl, N, K)
    assert dpl.numel() > (1 << 32)
    x = np.stack([q6ksynth.activation("outlier", K, 1600 + c) for c in range(nt)])
    qs, dd = oracle.quant_q8(x)
    y = run_mmvq(dpl, make_plane(qs, dd), N, K, nt)
    del dpl
    rng = np.random.default_rng(4243)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(N - 512, N),
                                     rng.integers(0, N, 512)]))
    raw_h = raw[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    del raw
    torch.cuda.empty_cache()
    y_or, A = oracle.mmvq(oracle.RAW, raw_h.reshape(-1), rows.size, K, qs, dd,
                          nthreads=oracle_threads())
    worst = check_y(y[:, rows], y_or, A, f"past 4 GiB N={N} K={K} nt={nt}")
    say(f"past 4 GiB N={N} K={K} nt={nt}: {rows.size} rows checked, max err/A = {worst:.3e}")


# The longest row the boundary accepts (K = 2^20, 4096 super-blocks: the generic
# stepping kernel), a few rows, one and several tokens.
@pytest.mark.parametrize("nt", [1, 3])
def test_longest_rows(nt):
    N, K = 7, 1 << 20
    raw = q6ksynth.raw_q6k(N, K, seed=77 + nt)
    dpl = dpl_from_raw(raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 1800 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_mmvq(dpl, make_plane(qs, d), N, K, nt)
    y_or, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d)
    check_y(y, y_or, A, f"K=2^20 nt={nt}")


@pytest.mark.parametrize("q0", [0, 1, 31, 33, 63])
@pytest.mark.parametrize("nbe,block", [(1, 0), (4, 3)])
def test_onehot_diagonal(q0, nbe, block):
    raw, qs, d16, expect = onehot_probe(q0, nbe=nbe, block=block)
    K = 256 * nbe
    y = run_mmvq(dpl_from_raw(raw, 256, K), make_plane(qs, d16), 256, K, 256)
    assert np.array_equal(y, expect.astype(np.float32))


@pytest.mark.parametrize("N", [1, 2, 3, 63, 64, 65, 255, 256, 257, 4097])
def test_row_counts(N):
    K, nt = 5120, 2
    raw = q6ksynth.raw_q6k(N, K, seed=N)
    x = np.stack([q6ksynth.activation("normal", K, 1100 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    y = run_mmvq(dpl_from_raw(raw, N, K), make_plane(qs, d), N, K, nt)
    y_or, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d)
    check_y(y, y_or, A, f"N={N}")


def test_zero_scale_rows_are_exactly_zero():
    N, K, nt = 40, 5120, 1
    raw = q6ksynth.raw_q6k(N, K, seed=1)
    blocks = raw.reshape(N, K // 256, 210)
    blocks[::3, :, 208:210] = 0                      # every third row: d = 0
    x = q6ksynth.activation("normal", K, 5)[None]
    qs, d = oracle.quant_q8(x)
    y = run_mmvq(dpl_from_raw(raw, N, K), make_plane(qs, d), N, K, 1)
    assert np.all(y[0, ::3] == 0)
    y_or, A = oracle.mmvq(oracle.RAW, raw, N, K, qs, d)
    check_y(y, y_or, A, "zero-scale rows")


# one wave per row; row pairs; rows shared by a workgroup (one token and four)
@pytest.mark.parametrize("N,K,nt", [(2048, 5120, 1), (8192, 5120, 4), (3584, 18944, 1),
                                    (3000, 13824, 4)])
def test_side_stream_and_repeat_calls_agree(N, K, nt):
    raw = q6ksynth.raw_q6k(N, K, seed=2)
    dpl = dpl_from_raw(raw, N, K)
    x = np.stack([q6ksynth.activation("outlier", K, 6 + c) for c in range(nt)])
    qs, d = oracle.quant_q8(x)
    plane = make_plane(qs, d)
    y1 = run_mmvq(dpl, plane, N, K, nt)
    s = torch.cuda.Stream()
    y2 = torch.empty((nt, N), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(3):
            q.mmvq_q6k_q8(dpl, plane, y2, N, K, nt)
    s.synchronize()
    assert np.array_equal(y1, y2.cpu().numpy())      # same kernel, same order: bitwise
