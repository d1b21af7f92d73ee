"""The producer -> GEMV chain (and the fused RMSNorm -> q8 -> GEMV call) captured
in a HIP graph and replayed.

The library queues plain kernel launches on the caller's stream (no allocation,
no memset, no synchronisation), so torch's graph capture records them. Every
replay is checked bitwise against eager execution of the same kernels, with new
inputs copied in eagerly and the stream synchronised between replays, and against
the oracle: the q8 plane bit for bit against the oracle quantizer of the replay's
own producer output (its input row for the plain quantizer), the GEMV outputs
against the oracle GEMV on the replay's own plane, and for Form B the SwiGLU output
against the oracle SwiGLU of the replay's gate and up totals (4 ulp) and its q8
plane against the oracle quantizer of that output.
"""
import numpy as np
import pytest
import torch

import oracle
import q6ksynth
import quantized_decode_gemv_amd as q
from gpu_util import (DEV, check_plane_exact, check_y_on_plane, dev_f32, dpl_from_raw, say,
                      split_plane, swiglu_tol)

pytestmark = pytest.mark.gpu


def _buffers(producer, K, nt):
    return dict(
        x=torch.empty((nt, K), dtype=torch.float32, device=DEV),
        gamma=dev_f32(q6ksynth.gamma(K, 5)),
        gate=torch.empty((nt, K), dtype=torch.float32, device=DEV),
        up=torch.empty((nt, K), dtype=torch.float32, device=DEV),
        yn=torch.empty((nt, K), dtype=torch.float32, device=DEV),
        plane=torch.empty(q.q8_plane_bytes(K, nt), dtype=torch.uint8, device=DEV),
        plane_out=torch.empty(max(q.q8_plane_bytes(2048, 1), 16), dtype=torch.uint8, device=DEV),
    )


def _step(producer, b, W, y, N, K, nt):
    if producer == "formb":   # rows [gate; up], the q8 plane of x as input
        q.quant_q8(b["x"], b["plane"], K, nt)
        q.mmvq_kq_gate_up_swiglu_q8(q.KQ_Q6_K, W, b["plane"], y.view(-1), b["yn"].view(-1)[:N // 2],
                                    b["plane_out"], N // 2, K)
        return
    if producer == "fused":
        q.mmvq_q6k_rmsnorm_q8(W, b["x"], b["gamma"], q6ksynth.RMS_EPS, b["yn"], b["plane"], y,
                              N, K, nt)
        return
    if producer == "rmsnorm":
        q.rmsnorm_quant_q8(b["x"], b["gamma"], q6ksynth.RMS_EPS, b["yn"], b["plane"], K, nt)
    elif producer == "swiglu":
        q.swiglu_quant_q8(b["gate"], b["up"], b["yn"], b["plane"], K, nt)
    else:
        q.quant_q8(b["x"], b["plane"], K, nt)
    q.mmvq_q6k_q8(W, b["plane"], y, N, K, nt)


def _fill(producer, b, K, nt, seed):
    if producer == "swiglu":
        g, u = (np.stack(a) for a in zip(*[q6ksynth.swiglu_pair(K, seed + c) for c in range(nt)]))
        b["gate"].copy_(torch.from_numpy(g))
        b["up"].copy_(torch.from_numpy(u))
    else:
        x = np.stack([q6ksynth.activation("outlier", K, seed + c) for c in range(nt)])
        b["x"].copy_(torch.from_numpy(x))


# the GEMV kinds: one wave per row, row pairs (8192 x 5120 at 4 tokens), the matrix-core
# tiles (49152 x 5120 at 4 tokens: buffer-to-LDS copies, counted waits and barriers),
# rows shared by a workgroup (3584 x 18944, 3000 x 13824 at 4 tokens), the generic
# stepping kernel
@pytest.mark.parametrize("producer,N,K,nt", [("rmsnorm", 4096, 5120, 1), ("rmsnorm", 2048, 5120, 4),
                                             ("rmsnorm", 8192, 5120, 4), ("rmsnorm", 49152, 5120, 4),
                                             ("swiglu", 1024, 13824, 1), ("swiglu", 3584, 18944, 1),
                                             ("quant", 64, 1024, 2), ("quant", 3000, 13824, 4),
                                             ("quant", 333, 256 * 97, 5),
                                             ("fused", 4096, 5120, 1), ("fused", 1024, 5120, 2),
                                             ("formb", 4096, 5120, 1)])
def test_graph_replays_match_eager(producer, N, K, nt):
    if N == 49152:
        assert q.mmvq_plan(N, K, nt, 256)["tiles"]
    raw = q6ksynth.raw_q6k(N, K, seed=N + K)
    W = dpl_from_raw(raw, N, K)
    b = _buffers(producer, K, nt)
    y = torch.empty((nt, N), dtype=torch.float32, device=DEV)
    _fill(producer, b, K, nt, 100)
    _step(producer, b, W, y, N, K, nt)          # warm: device tables filled before capture
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            _step(producer, b, W, y, N, K, nt)
    torch.cuda.synchronize()

    for rep in range(5):
        _fill(producer, b, K, nt, 200 + 10 * rep)   # eager input change between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = y.clone()
        plane_g = b["plane"].clone()
        out_g = b["plane_out"].clone()
        yn_g = b["yn"].clone()
        _step(producer, b, W, y, N, K, nt)          # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(b["plane"], plane_g), f"replay {rep}: q8 plane differs from eager"
        assert torch.equal(b["plane_out"], out_g), f"replay {rep}: output plane differs"
        assert torch.equal(y, got), f"replay {rep}: y differs from eager"
        _check_replay_vs_oracle(producer, b, raw, got, plane_g, out_g, yn_g, N, K, nt,
                                f"graph {producer} replay {rep}")
    say(f"graph {producer} N={N} K={K} nt={nt}: 5 replays bitwise equal to eager and "
        f"within the oracle's bounds")


def _check_replay_vs_oracle(producer, b, raw, y, plane, plane_out, yn, N, K, nt, what):
    qs, d = split_plane(plane, K, nt)
    if producer in ("quant", "formb"):
        src = b["x"].cpu().numpy()              # the plain quantizer's input row
    else:
        src = yn.cpu().numpy()                  # the producer's own output row
    check_plane_exact(src, qs, d, what + " q8")
    yh = y.cpu().numpy()
    check_y_on_plane(yh, raw, qs, d, N, K, what + " y")
    if producer == "formb":
        Nh = N // 2
        gu = yh.reshape(-1)
        sw = yn.cpu().numpy().reshape(-1)[:Nh]
        sw_or = oracle.swiglu(gu[None, :Nh], gu[None, Nh:])[0]
        tol = swiglu_tol(sw_or, gu[:Nh], gu[Nh:])
        assert np.all(np.abs(sw.astype(np.float64) - sw_or) <= tol), what + " swiglu"
        po = plane_out.cpu().numpy()
        check_plane_exact(sw[None], po[:Nh].view(np.int8)[None],
                          po[Nh:Nh + Nh // 16].view(np.uint16)[None], what + " q8 out")
