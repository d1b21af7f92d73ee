"""Pins for the q4_K / q5_K oracle (CPU only): the hand-worked layout, addressing and
scale-packing fixtures, closed forms, exact integer sums, brute force, and the
raw == split-plane invariant."""
import numpy as np
import pytest

import oracle
import q6ksynth
from golden_io import kq_code_addressing, kq_layout, kq_scale_bits
from kq_build import blank, block_info, set_code, set_d, set_scale_min

TYPES = [oracle.Q4_K, oracle.Q5_K]
NAMES = {oracle.Q4_K: "q4_K", oracle.Q5_K: "q5_K"}
LAYOUT = kq_layout()


def _ids(t):
    return NAMES[t]


# --- layout -------------------------------------------------------------------------

@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("nbe", [1, 2, 20, 54, 97])
def test_block_bytes_and_row_strides(qtype, nbe):
    info = LAYOUT["block"][NAMES[qtype]]
    assert oracle.kq_block_bytes(qtype) == info["bytes"]
    assert oracle.kq_row_stride(qtype, oracle.RAW, 256 * nbe) == nbe * info["bytes"]
    stride = oracle.kq_row_stride(qtype, oracle.DPL, 256 * nbe)
    assert stride == nbe * LAYOUT["plane"][NAMES[qtype]]["stride"] and stride % 16 == 0


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
def test_bad_shapes_rejected(qtype):
    for K in (0, 100, 255, 257):
        with pytest.raises(ValueError):
            oracle.kq_row_stride(qtype, oracle.DPL, K)
    with pytest.raises(ValueError):
        oracle.kq_block_bytes(14)


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("N,nbe", [(1, 1), (3, 4), (2, 20), (2, 54)])
def test_repack_places_every_field_in_its_plane(qtype, N, nbe):
    K = 256 * nbe
    raw = q6ksynth.raw_kq(qtype, N, K, seed=31 + N + nbe)
    dpl = oracle.kq_repack_dpl(qtype, raw, N, K).reshape(N, -1)
    info, plane = LAYOUT["block"][NAMES[qtype]], LAYOUT["plane"][NAMES[qtype]]
    B = info["bytes"]
    fields = [("codes", 128), ("scales", 12)] + ([("fifth", 32)] if info["fifth"] is not None else [])
    for r in range(N):
        for b in range(nbe):
            blk = raw[r, b * B:(b + 1) * B]
            for name, size in fields:
                got = dpl[r, plane[name] * nbe + b * size: plane[name] * nbe + (b + 1) * size]
                assert np.array_equal(got, blk[info[name]:info[name] + size]), (name, r, b)
            dm = dpl[r, plane["dm"] * nbe + 4 * b: plane["dm"] * nbe + 4 * b + 4]
            assert np.array_equal(dm[:2], blk[info["d"]:info["d"] + 2])
            assert np.array_equal(dm[2:], blk[info["dmin"]:info["dmin"] + 2])
    assert np.array_equal(oracle.kq_unpack_dpl(qtype, dpl, N, K).reshape(N, -1), raw)


# --- code addressing and scale packing ---------------------------------------------

@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("sub", kq_code_addressing(), ids=lambda u: "s%d" % u["s"])
@pytest.mark.parametrize("l", [0, 5, 15, 16, 31])
def test_code_addressing_matches_fixture(qtype, sub, l):
    """Perturb single code bytes / fifth bits of an all-zero block; exactly the
    element the hand-worked table names must change."""
    info = block_info(qtype)
    e = sub["first"] + l
    raw = blank(qtype, 1)
    i = info["codes"] + sub["window"] + l
    raw[0, i] = 0x09 if sub["nibble"] == "lo" else 0x90
    q, *_ = oracle.kq_decode(qtype, oracle.RAW, raw, 1, 256)
    expect = np.zeros(256, np.uint8)
    expect[e] = 9
    assert np.array_equal(q[0], expect)
    # the other nibble of the same byte belongs to the partner sub-block
    raw[0, i] = 0x90 if sub["nibble"] == "lo" else 0x09
    q, *_ = oracle.kq_decode(qtype, oracle.RAW, raw, 1, 256)
    assert q[0, e] == 0 and q[0].sum() == 9 and q[0, e ^ 32] == 9
    if info["fifth"] is not None:
        raw = blank(qtype, 1)
        raw[0, info["fifth"] + l] = 1 << sub["fifth_bit"]
        q, *_ = oracle.kq_decode(qtype, oracle.RAW, raw, 1, 256)
        expect = np.zeros(256, np.uint8)
        expect[e] = 16
        assert np.array_equal(q[0], expect)


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("bit", kq_scale_bits(), ids=lambda b: "b%d.%d" % (b[0], b[1]))
def test_scale_packing_matches_fixture(qtype, bit):
    """Each of the 96 packed bits lands in exactly the scale/min bit the table names."""
    byte, k, field, sub, dst = bit
    raw = blank(qtype, 1)
    raw[0, block_info(qtype)["scales"] + byte] = 1 << k
    _, sc, m, _, _ = oracle.kq_decode(qtype, oracle.RAW, raw, 1, 256)
    want_sc, want_m = np.zeros(8, np.uint8), np.zeros(8, np.uint8)
    (want_sc if field == "sc" else want_m)[sub] = 1 << dst
    assert np.array_equal(sc[0], want_sc) and np.array_equal(m[0], want_m)


def test_scale_packing_table_covers_every_field_bit_once():
    seen = {(f, s, b) for _, _, f, s, b in kq_scale_bits()}
    assert len(kq_scale_bits()) == 96 == len(seen)
    assert seen == {(f, s, b) for f in ("sc", "m") for s in range(8) for b in range(6)}


# --- the GEMV --------------------------------------------------------------------------

def _ones_q8(K, nt=1, d8=1.0):
    qs = np.ones((nt, K), np.int8)
    d16 = np.full((nt, K // 32), np.float16(d8).view(np.uint16), np.uint16)
    return qs, d16


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("code", [0, 1, 7, 15, 16, 31])
def test_closed_form_scale_term(qtype, code):
    # every code c, every scale v, no min, d = 1: y = v * c * K exactly
    if qtype == oracle.Q4_K and code > 15:
        pytest.skip("q4_K codes are 4 bits")
    nbe, v = 3, 5
    raw = blank(qtype, nbe)
    for b in range(nbe):
        set_d(qtype, raw[b], 1.0, 7.0)
        for s in range(8):
            set_scale_min(qtype, raw[b], s, v, 0)
        for e in range(256):
            set_code(qtype, raw[b], e, code)
    K = 256 * nbe
    qs, d16 = _ones_q8(K)
    y, A = oracle.kq_mmvq(qtype, oracle.RAW, raw.reshape(1, -1), 1, K, qs, d16)
    assert y[0, 0] == v * code * K and A[0, 0] == v * code * K


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
def test_closed_form_min_term(qtype):
    # codes 0, mins m_s = s + 1, dmin = 0.5, x8 all 1: y = -0.5 * 32 * sum(m) per block
    nbe = 2
    raw = blank(qtype, nbe)
    for b in range(nbe):
        set_d(qtype, raw[b], 3.0, 0.5)
        for s in range(8):
            set_scale_min(qtype, raw[b], s, 63, s + 1)
    K = 256 * nbe
    qs, d16 = _ones_q8(K, d8=2.0)
    y, A = oracle.kq_mmvq(qtype, oracle.RAW, raw.reshape(1, -1), 1, K, qs, d16)
    expect = -nbe * 0.5 * 2.0 * 32 * sum(range(1, 9))
    assert y[0, 0] == expect and A[0, 0] == -expect


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("q0", [1, 9, 15, 17, 31])
def test_onehot_diagonal(qtype, q0):
    """Row e holds code q0 at element e only (scale s + 1 for sub-block s, no min,
    d = 1); column e' is the one-hot activation at e'. Y[e'][e] = (s+1) * q0 on the
    diagonal, 0 elsewhere -- the element mapping and the activation alignment."""
    if qtype == oracle.Q4_K and q0 > 15:
        pytest.skip("q4_K codes are 4 bits")
    raw = blank(qtype, 256)
    for e in range(256):
        set_d(qtype, raw[e], 1.0, 1.0)
        for s in range(8):
            set_scale_min(qtype, raw[e], s, s + 1, 0)
        set_code(qtype, raw[e], e, q0)
    qs = np.eye(256, dtype=np.int8)
    d16 = np.full((256, 8), np.float16(1.0).view(np.uint16), np.uint16)
    y, _ = oracle.kq_mmvq(qtype, oracle.RAW, raw, 256, 256, qs, d16)
    expect = np.diag([(e // 32 + 1) * q0 for e in range(256)]).astype(np.float64)
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
def test_min_term_follows_subblock_of_activation(qtype):
    # row s has min s + 1 on sub-block s only; a one-hot activation at element e meets
    # it when e is in sub-block s: Y[e][s] = -(s + 1) exactly then, else 0
    raw = blank(qtype, 8)
    for s in range(8):
        set_d(qtype, raw[s], 1.0, 1.0)
        set_scale_min(qtype, raw[s], s, 0, s + 1)
    qs = np.eye(256, dtype=np.int8)
    d16 = np.full((256, 8), np.float16(1.0).view(np.uint16), np.uint16)
    y, _ = oracle.kq_mmvq(qtype, oracle.RAW, raw, 8, 256, qs, d16)
    expect = np.zeros((256, 8))
    for e in range(256):
        expect[e, e // 32] = -(e // 32 + 1)
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
@pytest.mark.parametrize("N,K,nt", [(5, 256, 1), (3, 1024, 2), (2, 5120, 3)])
def test_brute_force_and_exact(qtype, N, K, nt):
    raw = q6ksynth.raw_kq(qtype, N, K, seed=N * 13 + K)
    x = np.stack([q6ksynth.activation("outlier", K, 40 + c) for c in range(nt)])
    qs, d16 = oracle.quant_q8(x)
    y, A = oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, qs, d16)
    # brute force: dequantized weights times dequantized activations, fp64
    w = oracle.kq_dequant(qtype, oracle.RAW, raw, N, K)
    xd = qs.astype(np.float64) * np.repeat(d16.view(np.float16).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(xd @ w.T - y) <= 1e-12 * A)
    # the exact 128-bit sum: the fp64 sum is within n * 2^-53 * A of it
    ye = oracle.kq_mmvq_exact(qtype, oracle.RAW, raw, N, K, qs, d16)
    n = 2 * K // 32
    assert np.all(np.abs(ye - y) <= n * 2.0 ** -53 * A)
    # the split-plane layout gives the same result bit for bit
    dpl = oracle.kq_repack_dpl(qtype, raw, N, K)
    y2, A2 = oracle.kq_mmvq(qtype, oracle.DPL, dpl, N, K, qs, d16)
    assert np.array_equal(y, y2) and np.array_equal(A, A2)


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
def test_subdots_are_exact_code_dots(qtype):
    N, K = 4, 512
    raw = q6ksynth.raw_kq(qtype, N, K, seed=77)
    x = np.stack([q6ksynth.activation("normal", K, 78 + c) for c in range(2)])
    qs, _ = oracle.quant_q8(x)
    dots = oracle.kq_subdots(qtype, oracle.RAW, raw, N, K, qs)
    q, *_ = oracle.kq_decode(qtype, oracle.RAW, raw, N, K)
    want = np.einsum("rsk,tsk->trs", q.reshape(N, K // 32, 32).astype(np.int64),
                     qs.reshape(2, K // 32, 32).astype(np.int64))
    assert np.array_equal(dots, want)
    assert q.max() <= (15 if qtype == oracle.Q4_K else 31)


@pytest.mark.parametrize("qtype", TYPES, ids=_ids)
def test_special_cases(qtype):
    N, K = 3, 512
    raw = q6ksynth.raw_kq(qtype, N, K, seed=5)
    x = q6ksynth.activation("normal", K, 6)[None]
    qs, d16 = oracle.quant_q8(x)
    # zero activation -> exactly zero
    y, A = oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, np.zeros_like(qs), d16)
    assert not y.any()
    # d and dmin doubled (exact in fp16) -> y doubled exactly
    y1, _ = oracle.kq_mmvq(qtype, oracle.RAW, raw, N, K, qs, d16)
    raw2 = raw.reshape(N * 2, -1).copy()
    dm = raw2[:, :4].copy().view(np.float16) * np.float16(2)
    raw2[:, :4] = dm.view(np.uint8)
    y2, _ = oracle.kq_mmvq(qtype, oracle.RAW, raw2.reshape(N, -1), N, K, qs, d16)
    assert np.array_equal(y2, 2 * y1)
