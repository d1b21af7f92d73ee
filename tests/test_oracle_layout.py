"""Pins for the oracle's row layouts, repack and element decode (CPU only).

Each check compares the oracle with a printed value or a hand-worked fixture from
tests/golden/, never with the oracle itself.
"""
import numpy as np
import pytest

import oracle
import q6ksynth
from golden_io import dpl_layout, unit_addressing
from q6k_build import BLOCK, blank

LAYOUT = dpl_layout()


def test_dpl_stride_printed_example():
    # D4-4 §2: nbe 54 -> 11340 content bytes -> row stride 11344.
    K = 54 * 256
    assert oracle.row_stride(oracle.RAW, K) == LAYOUT["stride_nbe54_content"]
    assert oracle.row_stride(oracle.DPL, K) == LAYOUT["stride_nbe54"]
    assert oracle.row_stride(oracle.PAD224, K) == 54 * 224


@pytest.mark.parametrize("nbe", list(range(1, 130)) + [200, 592])
def test_dpl_stride_is_16_aligned_and_tight(nbe):
    s = oracle.row_stride(oracle.DPL, 256 * nbe)
    assert s % 16 == 0 and 0 <= s - 210 * nbe <= 15


@pytest.mark.parametrize("K", [0, -256, 100, 255, 257, 1000])
def test_bad_K_rejected(K):
    with pytest.raises(ValueError):
        oracle.row_stride(oracle.DPL, K)


@pytest.mark.parametrize("N,K", [(1, 256), (3, 1024), (7, 13824), (2, 18944)])
def test_repack_round_trip_and_zero_tail(N, K):
    raw = q6ksynth.raw_q6k(N, K, seed=17 + N)
    dpl = oracle.repack_dpl(raw, N, K)
    assert np.array_equal(oracle.unpack_dpl(dpl, N, K).reshape(N, -1), raw)
    nbe, stride = K // 256, oracle.row_stride(oracle.DPL, K)
    rows = dpl.reshape(N, stride)
    assert not rows[:, nbe * 210:].any(), "row tail pad must be zero"


def test_repack_sections_follow_printed_bases():
    # D4-4 §3.2 Excerpt A/B: field [a, b) of raw block i lands in its plane at
    # base*nbe + i*(b-a).
    N, K = 3, 5120
    nbe = K // 256
    raw = q6ksynth.raw_q6k(N, K, seed=5)
    dpl = oracle.repack_dpl(raw, N, K).reshape(N, -1)
    planes = [("raw_ql", LAYOUT["base_ql"]), ("raw_qh", LAYOUT["base_qh_per_nbe"]),
              ("raw_sc", LAYOUT["base_sc_per_nbe"]), ("raw_d", LAYOUT["base_d_per_nbe"])]
    for key, base in planes:
        a, b = LAYOUT[key]
        width = b - a
        for r in range(N):
            for i in range(nbe):
                src = raw[r, i * BLOCK + a:i * BLOCK + b]
                dst = dpl[r, base * nbe + i * width: base * nbe + (i + 1) * width]
                assert np.array_equal(src, dst), (key, r, i)


@pytest.mark.parametrize("N,K", [(4, 256), (5, 5120), (2, 18944)])
def test_decode_same_in_all_three_layouts(N, K):
    # D4-4 §2 "Why bitwise survives": the rearrangement is a pure byte move.
    raw = q6ksynth.raw_q6k(N, K, seed=99)
    a = oracle.decode(oracle.RAW, raw, N, K)
    b = oracle.decode(oracle.PAD224, oracle.pad224(raw, N, K), N, K)
    c = oracle.decode(oracle.DPL, oracle.repack_dpl(raw, N, K), N, K)
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)
    assert a[0].max() <= 63


def test_pad224_has_zero_pad():
    N, K = 2, 1024
    raw = q6ksynth.raw_q6k(N, K, seed=3)
    pad = oracle.pad224(raw, N, K).reshape(-1, 224)
    assert not pad[:, 210:].any()
    assert np.array_equal(pad[:, :210], raw.reshape(-1, 210))


@pytest.mark.parametrize("unit", unit_addressing(), ids=lambda u: "pair%d" % u["pair"])
@pytest.mark.parametrize("l", [0, 5, 15, 16, 31])
def test_element_addressing_matches_fixture(unit, l):
    """Perturb single bytes of an all-zero block; exactly the element the hand-worked
    table names must change, with the low/high field landing in its own bits."""
    K = 256
    e = unit["first"] + l
    raw = blank(1, 1)
    ql_i = unit["ql_off"] + l
    raw[0, ql_i] = 0x09 if unit["nibble"] == "lo" else 0x90
    q, _, _ = oracle.decode(oracle.RAW, raw, 1, K)
    expect = np.zeros(K, np.uint8)
    expect[e] = 9
    assert np.array_equal(q[0], expect)
    # the other nibble of the same byte belongs to another unit
    raw[0, ql_i] = 0x90 if unit["nibble"] == "lo" else 0x09
    q, _, _ = oracle.decode(oracle.RAW, raw, 1, K)
    assert q[0, e] == 0 and q[0].sum() == 9
    # high bits
    raw = blank(1, 1)
    raw[0, 128 + unit["qh_off"] + l] = 3 << unit["shift"]
    q, _, _ = oracle.decode(oracle.RAW, raw, 1, K)
    expect = np.zeros(K, np.uint8)
    expect[e] = 48
    assert np.array_equal(q[0], expect)


@pytest.mark.parametrize("unit", unit_addressing(), ids=lambda u: "pair%d" % u["pair"])
def test_scale_and_d_addressing_matches_fixture(unit):
    raw = blank(1, 1)
    raw[0, 192 + unit["sc_lo"]] = 5
    raw[0, 192 + unit["sc_hi"]] = np.array([-7], np.int8).view(np.uint8)[0]
    raw[0, 208], raw[0, 209] = 0x00, 0x3C
    _, sc, d = oracle.decode(oracle.RAW, raw, 1, 256)
    j = unit["first"] // 16
    assert sc[0, j] == 5 and sc[0, j + 1] == -7
    assert np.count_nonzero(sc) == 2
    assert d[0, 0] == 0x3C00


def test_dpl_decode_reads_printed_section_bases():
    # Build a dpl row by hand: marker values in each plane at the printed bases.
    nbe, K = 3, 768
    stride = oracle.row_stride(oracle.DPL, K)
    row = np.zeros(stride, np.uint8)
    for b in range(nbe):
        row[LAYOUT["base_sc_per_nbe"] * nbe + 16 * b: LAYOUT["base_sc_per_nbe"] * nbe + 16 * b + 16] = b + 1
        row[LAYOUT["base_d_per_nbe"] * nbe + 2 * b] = 0x00
        row[LAYOUT["base_d_per_nbe"] * nbe + 2 * b + 1] = 0x3C + b
        # element 0 of block b: low nibble of ql byte 0, field 0 of qh byte 0
        row[LAYOUT["base_ql"] + 128 * b] = 0x0A
        row[LAYOUT["base_qh_per_nbe"] * nbe + 64 * b] = 0x01
    q, sc, d = oracle.decode(oracle.DPL, row, 1, K)
    for b in range(nbe):
        assert q[0, 256 * b] == 0x1A
        assert np.all(sc[0, 16 * b:16 * b + 16] == b + 1)
        assert d[0, b] == 0x3C00 + (b << 8)
    assert np.count_nonzero(q) == nbe
