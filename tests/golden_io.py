"""Readers for the text fixtures under tests/golden/ (comments start with '#')."""
from __future__ import annotations

import numpy as np

from conftest import golden_path


def _lines(name):
    with open(golden_path(name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def unit_addressing():
    """-> list of dicts, one per unit (pair) of a super-block."""
    rows = []
    for line in _lines("q6k_unit_addressing.txt"):
        p, first, qlo, nib, qho, sh, slo, shi = line.split()
        rows.append(dict(pair=int(p), first=int(first), ql_off=int(qlo), nibble=nib,
                         qh_off=int(qho), shift=int(sh), sc_lo=int(slo), sc_hi=int(shi)))
    return rows


def dpl_layout():
    out = {}
    for line in _lines("dpl_layout.txt"):
        key, *vals = line.split()
        out[key] = [int(v) for v in vals] if len(vals) > 1 else int(vals[0])
    return out


def q8_cases():
    """-> list of (name, x float32[32], q int8[32], d16 int)."""
    cases, cur = [], None
    for line in _lines("q8_closed_form.txt"):
        tag, *vals = line.split()
        if tag == "case":
            cur = {"name": vals[0]}
            cases.append(cur)
        elif tag == "x":
            bits = np.zeros(32, np.uint32)
            bits[:len(vals)] = [int(v, 16) for v in vals]
            cur["x"] = bits.view(np.float32)
        elif tag == "q":
            q = np.zeros(32, np.int8)
            q[:len(vals)] = [int(v) for v in vals]
            cur["q"] = q
        elif tag == "d16":
            cur["d16"] = int(vals[0], 16)
    return [(c["name"], c["x"], c["q"], c["d16"]) for c in cases]


def kq_layout():
    """-> {"block": {type: dict}, "plane": {type: dict}} (offsets; None where absent)."""
    out = {"block": {}, "plane": {}}
    conv = lambda v: None if v == "-" else int(v)  # noqa: E731
    for line in _lines("kq_layout.txt"):
        kind, name, *vals = line.split()
        v = [conv(a) for a in vals]
        if kind == "block":
            out["block"][name] = dict(bytes=v[0], d=v[1], dmin=v[2], scales=v[3], fifth=v[4],
                                      codes=v[5])
        else:
            out["plane"][name] = dict(codes=v[0], fifth=v[1], scales=v[2], dm=v[3], stride=v[4])
    return out


def kq_code_addressing():
    rows = []
    for line in _lines("kq_code_addressing.txt"):
        s, first, win, nib, fb = line.split()
        rows.append(dict(s=int(s), first=int(first), window=int(win), nibble=nib,
                         fifth_bit=int(fb)))
    return rows


def kq_scale_bits():
    """-> list of (byte, bit, field, sub_block, dst_bit), one per packed bit."""
    out = []
    for line in _lines("kq_scale_bits.txt"):
        byte, lo, hi, field, sub, dst = line.split()
        for k in range(int(lo), int(hi) + 1):
            out.append((int(byte), k, field, int(sub), int(dst) + k - int(lo)))
    return out
