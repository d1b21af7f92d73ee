"""The C ABI on the CPU: exported symbols, argument validation, sizes, host repack.

No test here queues device work: every call with device pointers is given an
argument that validation rejects before any HIP call is made.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import q6ksynth
import quantized_decode_gemv_amd as q
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "q6kdpl.h")
E_SHAPE, E_NULL, E_ALIGN, E_ALIAS = -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[a-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    for n in ["repack_q6k_dpl", "rmsnorm_quant_q8", "mmvq_q6k_q8", "quant_q8", "swiglu_quant_q8",
              "repack_q6k_dpl_host", "unpack_q6k_dpl_host", "mmvq_q6k_q8_subdots",
              "q6k_strerror", "q6k_dpl_row_stride", "q8_plane_bytes"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    dll = ctypes.CDLL(q.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(dll, n)]
    assert not missing, missing


def test_version_and_errors_text():
    assert "gfx950" in q.q6k_version()
    for code in (0, -1, -2, -3, -4, -5, -99):
        assert q.lib().q6k_strerror(code)


@pytest.mark.parametrize("nbe", [1, 4, 20, 54, 74, 96, 97, 200, 4096])
def test_sizes_match_oracle(nbe):
    K = 256 * nbe
    assert q.q6k_dpl_row_stride(K) == oracle.row_stride(oracle.DPL, K)
    assert q.q6k_dpl_bytes(7, K) == 7 * oracle.row_stride(oracle.DPL, K)
    assert q.q6k_raw_bytes(7, K) == 7 * 210 * nbe
    assert q.q8_plane_bytes(K, 3) == 3 * K + 3 * (K // 32) * 2


@pytest.mark.parametrize("K", [0, -256, 100, 255, 257, 256 * 4097])
def test_bad_K_sizes_are_zero(K):
    assert q.q6k_dpl_row_stride(K) == 0 and q.q6k_dpl_bytes(1, K) == 0


def test_bad_sizes_are_zero():
    assert q.q6k_dpl_bytes(0, 256) == 0 and q.q6k_dpl_bytes(-1, 256) == 0
    assert q.q8_plane_bytes(48, 1) == 0 and q.q8_plane_bytes(64, 0) == 0
    assert q.q8_plane_bytes(64, 257) == 0 and q.q8_plane_bytes(64, 256) == 256 * 68


@pytest.mark.parametrize("N,K", [(1, 256), (5, 5120), (3, 18944), (2, 256 * 97)])
def test_host_repack_matches_oracle_and_round_trips(N, K):
    raw = q6ksynth.raw_q6k(N, K, seed=N + K)
    dpl = np.full(q.q6k_dpl_bytes(N, K), 0xEE, np.uint8)   # pad bytes must be overwritten
    q.repack_q6k_dpl_host(raw, dpl, N, K)
    assert np.array_equal(dpl, oracle.repack_dpl(raw, N, K))
    back = np.zeros_like(raw)
    q.unpack_q6k_dpl_host(dpl, back, N, K)
    assert np.array_equal(back, raw)


def test_host_repack_rejects_overlap_and_null():
    buf = np.zeros(4096, np.uint8)
    with pytest.raises(q.Q6kError) as e:
        q.repack_q6k_dpl_host(buf, buf.ctypes.data + 16, 1, 256)
    assert e.value.code == E_ALIAS
    with pytest.raises(q.Q6kError) as e:
        q.repack_q6k_dpl_host(None, buf, 1, 256)
    assert e.value.code == E_NULL


# Fake, never-dereferenced device addresses (validation rejects before any HIP call).
A, B, C, D = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _code(fn, *args):
    with pytest.raises(q.Q6kError) as e:
        fn(*args)
    return e.value.code


@pytest.mark.parametrize("N,K,nt", [(0, 256, 1), (-3, 256, 1), (1, 0, 1), (1, 255, 1),
                                    (1, 288, 1), (1, 256, 0), (1, 256, 257),
                                    (1, 256 * 4097, 1), (2 ** 30 + 1, 256, 1)])
def test_mmvq_rejects_bad_shapes(N, K, nt):
    assert _code(q.mmvq_q6k_q8, A, B, C, N, K, nt, 0) == E_SHAPE
    assert _code(q.mmvq_q6k_q8_subdots, A, B, C, N, K, nt, 0) == E_SHAPE


def test_mmvq_rejects_null_misaligned_and_aliased():
    assert _code(q.mmvq_q6k_q8, None, B, C, 4, 256, 1, 0) == E_NULL
    assert _code(q.mmvq_q6k_q8, A, None, C, 4, 256, 1, 0) == E_NULL
    assert _code(q.mmvq_q6k_q8, A, B, None, 4, 256, 1, 0) == E_NULL
    assert _code(q.mmvq_q6k_q8, A + 8, B, C, 4, 256, 1, 0) == E_ALIGN
    assert _code(q.mmvq_q6k_q8, A, B + 4, C, 4, 256, 1, 0) == E_ALIGN
    assert _code(q.mmvq_q6k_q8, A, B, C + 2, 4, 256, 1, 0) == E_ALIGN
    # y overlapping the weights or the q8 plane
    assert _code(q.mmvq_q6k_q8, A, B, A + 16, 4, 256, 1, 0) == E_ALIAS
    assert _code(q.mmvq_q6k_q8, A, B, B + 32, 4, 256, 1, 0) == E_ALIAS
    assert _code(q.mmvq_q6k_q8, A, B, A - 16, 8, 256, 1, 0) == E_ALIAS
    assert _code(q.mmvq_q6k_q8_subdots, A, B, B, 4, 256, 1, 0) == E_ALIAS


def test_producers_reject_bad_arguments():
    assert _code(q.quant_q8, A, B, 48, 1, 0) == E_SHAPE
    assert _code(q.quant_q8, A, B, 64, 0, 0) == E_SHAPE
    assert _code(q.quant_q8, None, B, 64, 1, 0) == E_NULL
    assert _code(q.quant_q8, A + 4, B, 64, 1, 0) == E_ALIGN
    assert _code(q.quant_q8, A, A + 64, 64, 1, 0) == E_ALIAS
    assert _code(q.rmsnorm_quant_q8, A, B, 1e-6, C, D, 40, 1, 0) == E_SHAPE
    assert _code(q.rmsnorm_quant_q8, A, None, 1e-6, C, D, 64, 1, 0) == E_NULL
    assert _code(q.rmsnorm_quant_q8, A, B, 1e-6, C + 8, D, 64, 1, 0) == E_ALIGN
    assert _code(q.rmsnorm_quant_q8, A, B, 1e-6, A, D, 64, 1, 0) == E_ALIAS
    assert _code(q.rmsnorm_quant_q8, A, B, 1e-6, C, C + 16, 64, 1, 0) == E_ALIAS
    assert _code(q.rmsnorm_quant_q8, A, B, 1e-6, C, B, 64, 1, 0) == E_ALIAS


def test_swiglu_producer_rejects_bad_arguments():
    assert _code(q.swiglu_quant_q8, A, B, C, D, 40, 1, 0) == E_SHAPE
    assert _code(q.swiglu_quant_q8, A, B, C, D, 64, 0, 0) == E_SHAPE
    assert _code(q.swiglu_quant_q8, A, None, C, D, 64, 1, 0) == E_NULL
    assert _code(q.swiglu_quant_q8, A, B + 4, C, D, 64, 1, 0) == E_ALIGN
    # y overlapping g or u partially (not exactly in place), q8 overlapping anything
    assert _code(q.swiglu_quant_q8, A, B, A + 16, D, 64, 1, 0) == E_ALIAS
    assert _code(q.swiglu_quant_q8, A, B, B - 16, D, 64, 1, 0) == E_ALIAS
    assert _code(q.swiglu_quant_q8, A, B, C, A + 32, 64, 1, 0) == E_ALIAS
    assert _code(q.swiglu_quant_q8, A, B, C, C, 64, 1, 0) == E_ALIAS


def test_device_repack_rejects_bad_arguments():
    assert _code(q.repack_q6k_dpl, A, B, 1, 100, 0) == E_SHAPE
    assert _code(q.repack_q6k_dpl, A, None, 1, 256, 0) == E_NULL
    assert _code(q.repack_q6k_dpl, A, B + 1, 1, 256, 0) == E_ALIGN
    assert _code(q.repack_q6k_dpl, A, A + 64, 1, 256, 0) == E_ALIAS


@pytest.mark.parametrize("nbe", list(range(1, 121)) + [200, 592, 4096])
@pytest.mark.parametrize("nt", [1, 2, 4, 5, 9])
def test_plan_covers_every_row_length(nbe, nt):
    # every nbe reaches a kernel whose chunk count per lane covers the whole row
    p = q.mmvq_plan(1000, 256 * nbe, nt, 256)
    span = 256 if p["shared"] else 64
    assert p["cpl"] * span >= 8 * nbe > (p["cpl"] - 1) * span
    assert p["unrolled"] == (8 * nbe <= 12 * 64)
    assert p["launches"] == -(-nt // 4)
    assert p["act_mode"] in (0, 1, 2)
    assert p["grid"] >= 1 and p["depth"] in (1, 2, 3)


@pytest.mark.parametrize("qtype", [14, 12, 13])
@pytest.mark.parametrize("nbe", [20, 40, 47, 48, 49, 54, 74, 96, 97])
@pytest.mark.parametrize("N", [1, 3584, 5120, 8192, 131072, 131073, 152064])
@pytest.mark.parametrize("nt", [1, 2, 3, 4, 5])
def test_plan_shared_rows_rule(qtype, nbe, N, nt):
    # the workgroup-shared rows: chunks per lane (one wave per row) 7..12, or 6 from
    # 3 tokens; at one token q6_K only below 4 rows per wave of the one-wave grid;
    # at most 256 rows per workgroup
    cpl = -(-8 * nbe // 64)
    n = min(nt, 4)
    p = q.mmvq_plan(N, 256 * nbe, nt, 256, qtype)
    if not (7 <= cpl <= 12 or (cpl == 6 and n >= 3)):
        assert not p["shared"]
        return
    wpc = 2 if -(-cpl // 4) <= 2 else 1
    if -(-N // (256 * wpc)) > 256:
        assert not p["shared"]
        return
    if n == 1 and qtype == 14:
        assert p["shared"] == (N < 4 * 4 * 256 * (2 if cpl >= 9 else 1))
        if not p["shared"]:
            return
    assert p["shared"] and p["cpl"] == -(-cpl // 4)
    R = -(-N // (256 * wpc))
    assert p["grid"] == -(-N // R) and p["act_mode"] == 1 and p["depth"] == (2 if wpc == 2 else 3)


@pytest.mark.parametrize("qtype", [14, 12, 13])
@pytest.mark.parametrize("nbe", list(range(1, 41)))
@pytest.mark.parametrize("nt", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("N", [1000, 4094, 4095, 152064])
def test_plan_pairs_rule(qtype, nbe, nt, N):
    # two rows per wave at 2..4 tokens (per launch) when a row has an odd multiple of
    # 32 chunks, at most 3 chunks per lane, and at least two pairs per wave of the
    # grid (one workgroup per CU: 1024 waves on 256 CUs)
    # q6_K rows of 20 super-blocks at 3 or 4 tokens take the matrix-core tiles instead
    # when there are enough tiles of 16 rows (4 tokens: 12 per CU, 3 tokens: 24; one
    # workgroup per CU, two tile buffers)
    p = q.mmvq_plan(N, 256 * nbe, nt, 256, qtype)
    tiles = (qtype == 14 and nbe == 20 and min(nt, 4) >= 3
             and -(-N // 16) >= (12 if min(nt, 4) == 4 else 24) * 256)
    assert p["tiles"] == tiles
    if tiles:
        assert not p["paired"] and p["grid"] == min(-(-N // 16), 256)
        assert p["depth"] == 2 and p["act_mode"] == 1 and p["unrolled"]
        return
    expect = (min(nt, 4) >= 2 and (8 * nbe) % 64 == 32 and -(-8 * nbe // 64) <= 3
              and (N + 1) // 2 >= 2048)
    assert p["paired"] == expect
    if expect:
        pairs = (N + 1) // 2
        assert p["cpl"] == -(-8 * nbe // 64) and p["grid"] == min(-(-pairs // 4), 256)
        assert p["depth"] == 2 and p["act_mode"] == 1


@pytest.mark.parametrize("num_cu", [256, 80, 304])
@pytest.mark.parametrize("nt", [2, 3, 4, 5, 8])
def test_plan_tiles_threshold(num_cu, nt):
    # the tiles take q6_K K = 5120 from 12 tiles of 16 rows per CU at 4 tokens and 24 at
    # 3 (per launch of up to 4 tokens); one row fewer keeps the row pairs
    n = min(nt, 4)
    if n < 3:
        assert not q.mmvq_plan(1 << 20, 5120, nt, num_cu)["tiles"]
        return
    first = 16 * (12 if n == 4 else 24) * num_cu
    at, below = q.mmvq_plan(first, 5120, nt, num_cu), q.mmvq_plan(first - 16, 5120, nt, num_cu)
    assert at["tiles"] and at["grid"] == num_cu and not below["tiles"]
    assert q.mmvq_plan(first - 15, 5120, nt, num_cu)["tiles"]
    assert not q.mmvq_plan(first, 5120, nt, num_cu, 12)["tiles"]
    assert not q.mmvq_plan(first, 4864, nt, num_cu)["tiles"]


@pytest.mark.parametrize("N", [1, 2, 3, 63, 64, 65, 1023, 1024, 1025, 4096, 152064])
@pytest.mark.parametrize("nt", [1, 2, 4])
def test_plan_grid_is_whole_cus_or_one_wave_per_row(N, nt):
    p = q.mmvq_plan(N, 5120, nt, 256)
    # 16-row tiles at 4 tokens from 12 tiles per CU: one workgroup per CU
    assert p["tiles"] == (nt == 4 and -(-N // 16) >= 12 * 256)
    if p["tiles"]:
        assert p["grid"] == min(-(-N // 16), 256)
        return
    # one wave per row, or per pair of rows (K = 5120 at several tokens, enough rows)
    assert p["paired"] == (nt >= 2 and (N + 1) // 2 >= 2 * 1024)
    units = -(-N // 2) if p["paired"] else N
    waves_needed = -(-units // 4)
    assert p["grid"] == waves_needed or (p["grid"] % 256 == 0 and p["grid"] < waves_needed)


def test_fused_rmsnorm_mmvq_rejects_bad_arguments():
    E = 0x50000000
    f = q.mmvq_q6k_rmsnorm_q8
    # weights need K % 256 (the producers alone take K % 32)
    assert _code(f, A, B, C, 1e-6, None, D, E, 4, 288, 1, 0) == E_SHAPE
    assert _code(f, A, B, C, 1e-6, None, D, E, 0, 256, 1, 0) == E_SHAPE
    assert _code(f, A, B, C, 1e-6, None, D, E, 4, 256, 0, 0) == E_SHAPE
    assert _code(f, A, B, C, 1e-6, None, D, E, 4, 256, 257, 0) == E_SHAPE
    for i in range(3):
        args = [A, B, C]
        args[i] = None
        assert _code(f, *args, 1e-6, None, D, E, 4, 256, 1, 0) == E_NULL
    assert _code(f, A, B, C, 1e-6, None, None, E, 4, 256, 1, 0) == E_NULL
    assert _code(f, A, B, C, 1e-6, None, D, None, 4, 256, 1, 0) == E_NULL
    assert _code(f, A + 8, B, C, 1e-6, None, D, E, 4, 256, 1, 0) == E_ALIGN
    assert _code(f, A, B, C, 1e-6, E + 0x1000 + 4, D, E, 4, 256, 1, 0) == E_ALIGN
    assert _code(f, A, B, C, 1e-6, None, D + 2, E, 4, 256, 1, 0) == E_ALIGN
    # every output against every input and the other outputs; xn optional
    assert _code(f, A, B, C, 1e-6, None, A + 16, E, 4, 256, 1, 0) == E_ALIAS      # q8 / w
    assert _code(f, A, B, C, 1e-6, None, D, B + 16, 4, 256, 1, 0) == E_ALIAS      # y / x
    assert _code(f, A, B, C, 1e-6, C, D, E, 4, 256, 1, 0) == E_ALIAS              # xn / gamma
    assert _code(f, A, B, C, 1e-6, D - 512, D, E, 4, 256, 1, 0) == E_ALIAS        # xn / q8
    assert _code(f, A, B, C, 1e-6, None, D, D + 32, 4, 256, 1, 0) == E_ALIAS      # y / q8


@pytest.mark.parametrize("nbe", [1, 8, 9, 16, 17, 20, 24, 25, 40, 48, 49, 54, 74, 96, 97, 200])
@pytest.mark.parametrize("nt", [1, 2, 3, 4, 5, 8, 9])
def test_fused_rmsnorm_mmvq_shape_rule(nbe, nt):
    # one kernel for one token with at most 6 low-bit chunks per lane (K <= 12288),
    # where the GEMV keeps the activation operands in registers
    K = 256 * nbe
    expect = nt == 1 and nbe <= 48
    assert q.rmsnorm_mmvq_fused(1000, K, nt) == expect
    if expect:
        assert q.mmvq_plan(1000, K, nt, 256)["hoist"]


# --- q4_K / q5_K by weight type ------------------------------------------------------

KQ_TYPES = [q.KQ_Q4_K, q.KQ_Q5_K]


@pytest.mark.parametrize("qtype", KQ_TYPES)
@pytest.mark.parametrize("nbe", [1, 4, 20, 54, 97])
def test_kq_sizes_match_oracle(qtype, nbe):
    K = 256 * nbe
    assert q.kq_block_bytes(qtype) == oracle.kq_block_bytes(qtype)
    assert q.kq_dpl_row_stride(qtype, K) == oracle.kq_row_stride(qtype, oracle.DPL, K)
    assert q.kq_dpl_bytes(qtype, 7, K) == 7 * oracle.kq_row_stride(qtype, oracle.DPL, K)
    assert q.kq_raw_bytes(qtype, 7, K) == 7 * oracle.kq_row_stride(qtype, oracle.RAW, K)


def test_kq_q6k_type_equals_the_q6k_entries():
    for K in (256, 5120, 18944):
        assert q.kq_dpl_row_stride(q.KQ_Q6_K, K) == q.q6k_dpl_row_stride(K)
        assert q.kq_dpl_bytes(q.KQ_Q6_K, 3, K) == q.q6k_dpl_bytes(3, K)
        assert q.kq_raw_bytes(q.KQ_Q6_K, 3, K) == q.q6k_raw_bytes(3, K)
    assert q.kq_block_bytes(q.KQ_Q6_K) == 210


@pytest.mark.parametrize("qtype", KQ_TYPES)
@pytest.mark.parametrize("N,K", [(1, 256), (5, 5120), (3, 13824), (2, 256 * 97)])
def test_kq_host_repack_matches_oracle_and_round_trips(qtype, N, K):
    raw = q6ksynth.raw_kq(qtype, N, K, seed=N + K + qtype)
    dpl = np.full(q.kq_dpl_bytes(qtype, N, K), 0xEE, np.uint8)
    q.repack_kq_dpl_host(qtype, raw, dpl, N, K)
    assert np.array_equal(dpl, oracle.kq_repack_dpl(qtype, raw, N, K))
    back = np.zeros_like(raw)
    q.unpack_kq_dpl_host(qtype, dpl, back, N, K)
    assert np.array_equal(back, raw)


def test_kq_host_repack_q6k_type_matches_q6k_repack():
    N, K = 3, 5120
    raw = q6ksynth.raw_q6k(N, K, seed=9)
    a = np.zeros(q.q6k_dpl_bytes(N, K), np.uint8)
    b = np.zeros_like(a)
    q.repack_q6k_dpl_host(raw, a, N, K)
    q.repack_kq_dpl_host(q.KQ_Q6_K, raw, b, N, K)
    assert np.array_equal(a, b)


E_TYPE = -6


@pytest.mark.parametrize("bad", [0, 11, 15, -1, 2])
def test_kq_rejects_unknown_types(bad):
    assert q.kq_block_bytes(bad) == 0 and q.kq_dpl_row_stride(bad, 256) == 0
    assert q.kq_dpl_bytes(bad, 1, 256) == 0 and q.kq_raw_bytes(bad, 1, 256) == 0
    assert _code(q.mmvq_kq_q8, bad, A, B, C, 4, 256, 1, 0) == E_TYPE
    assert _code(q.repack_kq_dpl, bad, A, B, 1, 256, 0) == E_TYPE
    assert _code(q.mmvq_kq_q8_subdots, bad, A, B, C, 4, 256, 1, 0) == E_TYPE
    assert _code(q.mmvq_kq_rmsnorm_q8, bad, A, B, C, 1e-6, None, D, 0x50000000, 4, 256, 1,
                 0) == E_TYPE
    buf = np.zeros(4096, np.uint8)
    assert _code(q.repack_kq_dpl_host, bad, buf[:2048], buf[2048:], 1, 256) == E_TYPE
    assert _code(q.unpack_kq_dpl_host, bad, buf[:2048], buf[2048:], 1, 256) == E_TYPE


@pytest.mark.parametrize("qtype", KQ_TYPES)
def test_kq_gemv_rejects_bad_arguments(qtype):
    f = q.mmvq_kq_q8
    assert _code(f, qtype, A, B, C, 4, 288, 1, 0) == E_SHAPE
    assert _code(f, qtype, A, B, C, 0, 256, 1, 0) == E_SHAPE
    assert _code(f, qtype, None, B, C, 4, 256, 1, 0) == E_NULL
    assert _code(f, qtype, A + 8, B, C, 4, 256, 1, 0) == E_ALIGN
    assert _code(f, qtype, A, B, A + 16, 4, 256, 1, 0) == E_ALIAS
    # the weight extent is the type's: a y just past a q4_K matrix is fine for the
    # length check of q4_K but inside the bigger q5_K one
    n = q.kq_dpl_bytes(q.KQ_Q4_K, 4, 256)
    if qtype == q.KQ_Q5_K:
        assert _code(f, qtype, A, B, A + n, 4, 256, 1, 0) == E_ALIAS
    assert _code(q.mmvq_kq_q8_subdots, qtype, A, B, B, 4, 256, 1, 0) == E_ALIAS
    assert _code(q.repack_kq_dpl, qtype, A, A + 64, 1, 256, 0) == E_ALIAS


def test_form_b_rejects_bad_arguments():
    f = q.mmvq_kq_gate_up_swiglu_q8
    E, F_ = 0x50000000, 0x60000000
    t = q.KQ_Q4_K
    assert _code(f, 11, A, B, C, None, D, 64, 256, 1, 0) == E_TYPE
    assert _code(f, t, A, B, C, None, D, 48, 256, 1, 0) == E_SHAPE      # Nh % 32
    assert _code(f, t, A, B, C, None, D, 64, 256, 2, 0) == E_SHAPE      # one token only
    assert _code(f, t, A, B, C, None, D, 64, 288, 1, 0) == E_SHAPE      # K % 256
    assert _code(f, t, A, B, C, None, D, 0, 256, 1, 0) == E_SHAPE
    assert _code(f, t, None, B, C, None, D, 64, 256, 1, 0) == E_NULL
    assert _code(f, t, A, B, None, None, D, 64, 256, 1, 0) == E_NULL
    assert _code(f, t, A, B, C, None, None, 64, 256, 1, 0) == E_NULL
    assert _code(f, t, A, B, C + 4, None, D, 64, 256, 1, 0) == E_ALIGN
    assert _code(f, t, A, B, C, E + 8, D, 64, 256, 1, 0) == E_ALIGN
    assert _code(f, t, A, B, A + 16, None, D, 64, 256, 1, 0) == E_ALIAS   # gu / w
    assert _code(f, t, A, B, C, None, B + 16, 64, 256, 1, 0) == E_ALIAS   # q8_out / q8_in
    assert _code(f, t, A, B, C, C + 256, D, 64, 256, 1, 0) == E_ALIAS    # y / gu
    assert _code(f, t, A, B, C, None, C + 496, 64, 256, 1, 0) == E_ALIAS  # q8_out / gu
    assert q.gate_up_swiglu_fused(13824, 5120) and not q.gate_up_swiglu_fused(64, 256 * 49)
    with pytest.raises(q.Q6kError):
        q.gate_up_swiglu_fused(48, 256)


def test_read_probe_library_loads_and_rejects_bad_arguments():
    # the measurement probe (bench.py --read-ceiling) is a library of its own; its
    # argument checks run on the host before any GPU call
    import ctypes
    from quantized_decode_gemv_amd import build as libbuild
    lib = ctypes.CDLL(libbuild.PROBE_LIB)
    f = lib.q6k_read_probe
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p]
    good = 0x10000000
    assert f(None, 1 << 20, 2, 256, good, None) == -1          # no buffer
    assert f(good, 1 << 20, 2, 256, None, None) == -1          # no sink
    assert f(good, 4095, 2, 256, good, None) == -1             # less than one row
    assert f(good, 1 << 20, 0, 256, good, None) == -1          # depth 1..4
    assert f(good, 1 << 20, 5, 256, good, None) == -1
    assert f(good, 1 << 20, 2, 0, good, None) == -1            # no workgroups
    assert f(good + 8, 1 << 20, 2, 256, good, None) == -1      # 16-B alignment
