"""GPU coverage sweep: a GEMV that skips any unit of any row shows an exact deficit.

Every code 33 (q - 32 = 1), every scale 1, d = 1.0; every activation 1 with scale
1.0: each output is exactly K in f32. The pages' dispatch bug dropped units
512..591 of each 592-unit row (D4-2 §2); here every row length, row count and
token count must produce exactly K.
"""
import numpy as np
import pytest
import torch

import quantized_decode_gemv_amd as q
from gpu_util import DEV, dev_u8, say
from q6k_build import blank

pytestmark = pytest.mark.gpu

NBE = list(range(1, 81)) + [96, 97, 128, 200]
NS = [1, 2, 3, 63, 64, 65, 255, 256, 257, 4097]


def _ones_dpl(N, nbe):
    K = 256 * nbe
    row = blank(1, nbe, ql=0x11, qh=0xAA, sc=1, d_bits=0x3C00)
    dpl_row = torch.empty(q.q6k_dpl_bytes(1, K), dtype=torch.uint8, device=DEV)
    q.repack_q6k_dpl(dev_u8(row), dpl_row, 1, K)
    return dpl_row.repeat(N)


def _ones_plane(K, nt):
    qs = np.ones(nt * K, np.int8).view(np.uint8)
    d16 = np.full(nt * (K // 32), 0x3C00, np.uint16).view(np.uint8)
    return dev_u8(np.concatenate([qs, d16]))


@pytest.mark.parametrize("nbe", NBE)
def test_every_unit_counted(nbe):
    K = 256 * nbe
    say(f"coverage nbe={nbe}")
    for N in NS:
        dpl = _ones_dpl(N, nbe)
        for nt in (1, 2, 3, 4, 5):
            plane = _ones_plane(K, nt)
            y = torch.zeros((nt, N), dtype=torch.float32, device=DEV)
            q.mmvq_q6k_q8(dpl, plane, y, N, K, nt)
            yh = y.cpu().numpy()
            bad = np.argwhere(yh != K)
            assert bad.size == 0, f"nbe={nbe} N={N} nt={nt}: {len(bad)} outputs != K, e.g. {bad[:3]} -> {yh[tuple(bad[0])]}"


@pytest.mark.parametrize("nbe", [1, 20, 54, 74])
def test_every_unit_counted_lm_head_rows(nbe):
    N, K = 152064, 256 * nbe
    say(f"coverage N={N} nbe={nbe}")
    dpl = _ones_dpl(N, nbe)
    for nt in (1, 4, 5):
        y = torch.zeros((nt, N), dtype=torch.float32, device=DEV)
        q.mmvq_q6k_q8(dpl, _ones_plane(K, nt), y, N, K, nt)
        assert bool((y == K).all())
