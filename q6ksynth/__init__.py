"""Seeded synthetic inputs for the q6_K (and q4_K / q5_K) x q8 decode GEMV.

This module is shared by the oracle-side tests and the HIP-side tests and
benchmark. It holds none of the method's arithmetic: it draws random bytes and
random floats in the shapes and distributions of the workloads and places them
at the byte positions of a GGUF super-block, nothing more:
  q6_K (210 B): 128 B low bits, 64 B high bits, 16 int8 sub-block scales, fp16
    scale at byte 208; uniform low/high bytes give codes uniform in 0..63;
  q4_K (144 B): fp16 d and dmin at 0 and 2, 12 bytes of packed 6-bit scales and
    mins at 4, 128 code bytes at 16; q5_K (176 B): the same with 32 fifth-bit
    bytes at 16 and the code bytes at 48. Uniform bytes give uniform codes,
    scales and mins.
Activations are N(0,1) rows (with or without outliers) and the gate/up row pairs
that the SwiGLU producer consumes; SwiGLU itself is computed by the path (and by
the oracle), not here.

Scales are drawn as fp16(|N(0,1)| * 1e-3) rather than random bit patterns, so no
NaN or inf can appear (random fp16 bits make NaN != NaN comparisons look like
differences; D4-4 §3.3, "The NaN trap").
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BLOCK_BYTES = 210          # one q6_K super-block of 256 weights
QL_BYTES, QH_BYTES, SC_BYTES = 128, 64, 16
Q4_K, Q5_K, Q6_K = 12, 13, 14          # GGUF type ids
KQ_BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210}


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int             # 1-based workload number, used in the seeds
    name: str
    N: int                 # output rows
    K: int                 # input features (multiple of 256)
    nt: tuple              # token columns exercised
    act: str               # "normal" | "outlier" | "gate_up" (a gate/up pair per column)
    producer: str          # "quant" (standalone q8) | "rmsnorm" (fused RMSNorm -> q8)
                           # | "swiglu" (fused SwiGLU -> q8 from gate/up rows)
    qtype: int = Q6_K      # weight type (GGUF type id)

    @property
    def nbe(self) -> int:
        return self.K // 256

    @property
    def content_bytes(self) -> int:
        return self.N * self.nbe * KQ_BLOCK_BYTES[self.qtype]


WORKLOADS = {
    "tiny": Workload(1, "tiny", 64, 1024, (1,), "normal", "quant"),
    "attn_v": Workload(2, "attn_v", 1024, 5120, (1,), "outlier", "rmsnorm"),
    "ffn_down": Workload(3, "ffn_down", 5120, 13824, (1,), "gate_up", "swiglu"),
    "tall_k": Workload(4, "tall_k", 3584, 18944, (1,), "gate_up", "swiglu"),
    "lm_head": Workload(5, "lm_head", 152064, 5120, (1, 4), "outlier", "rmsnorm"),
    # q4_K / q5_K siblings on the same decode step: the fused gate+up matrix (the
    # pages' 27648 x 5120 q4_K probe shape) and the down projection (13824 -> 5120)
    "q4k_gate_up": Workload(6, "q4k_gate_up", 27648, 5120, (1, 4), "outlier", "rmsnorm", Q4_K),
    "q4k_down": Workload(7, "q4k_down", 5120, 13824, (1,), "gate_up", "swiglu", Q4_K),
    "q5k_gate_up": Workload(8, "q5k_gate_up", 27648, 5120, (1, 4), "outlier", "rmsnorm", Q5_K),
    "q5k_down": Workload(9, "q5k_down", 5120, 13824, (1,), "gate_up", "swiglu", Q5_K),
}

RMS_EPS = 1e-6


def weight_seed(w: Workload) -> int:
    return 1000 * w.index


def act_seed(w: Workload, column: int) -> int:
    return 1000 * w.index + 1 + column


def gamma_seed(w: Workload) -> int:
    return 1000 * w.index + 999


def _random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    """n uniform random bytes: the generator's raw 64-bit outputs, little-endian."""
    words = rng.bit_generator.random_raw((n + 7) // 8)
    return words.astype("<u8", copy=False).view(np.uint8)[:n]


def raw_q6k(N: int, K: int, seed: int) -> np.ndarray:
    """Random raw GGUF q6_K rows, uint8 [N, (K/256)*210].

    Low/high bit bytes are uniform random bytes; each int8 sub-block scale is a
    uniform byte masked to 6 bits minus 32 (exactly uniform on [-32, 31]); the fp16
    super-block scale is fp16(|N(0,1)| * 1e-3)."""
    assert K > 0 and K % 256 == 0 and N >= 0
    nbe = K // 256
    rng = np.random.default_rng(seed)
    nblk = N * nbe
    out = np.empty((nblk, BLOCK_BYTES), np.uint8)
    out[:, :QL_BYTES + QH_BYTES] = _random_bytes(rng, nblk * (QL_BYTES + QH_BYTES)).reshape(
        nblk, QL_BYTES + QH_BYTES)
    sc = (_random_bytes(rng, nblk * SC_BYTES) & 63).astype(np.int16) - 32
    out[:, 192:208] = sc.astype(np.int8).view(np.uint8).reshape(nblk, SC_BYTES)
    d = (np.abs(rng.standard_normal(nblk)) * 1e-3).astype(np.float16)
    out[:, 208:210] = d.view(np.uint8).reshape(nblk, 2)
    return out.reshape(N, nbe * BLOCK_BYTES)


def raw_kq(qtype: int, N: int, K: int, seed: int) -> np.ndarray:
    """Random raw GGUF q4_K / q5_K rows, uint8 [N, (K/256)*block bytes].

    Code, fifth-bit and packed scale/min bytes are uniform random bytes; d and dmin
    are fp16(|N(0,1)| * 1e-3) each."""
    assert qtype in (Q4_K, Q5_K) and K > 0 and K % 256 == 0 and N >= 0
    nbe, B = K // 256, KQ_BLOCK_BYTES[qtype]
    rng = np.random.default_rng(seed)
    nblk = N * nbe
    out = np.empty((nblk, B), np.uint8)
    out[:, 4:] = _random_bytes(rng, nblk * (B - 4)).reshape(nblk, B - 4)
    dm = (np.abs(rng.standard_normal((nblk, 2))) * 1e-3).astype(np.float16)
    out[:, 0:4] = dm.view(np.uint8).reshape(nblk, 4)
    return out.reshape(N, nbe * B)


def activation(kind: str, K: int, seed: int) -> np.ndarray:
    """One float32 activation row of length K ("normal" or "outlier")."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal(K, dtype=np.float32)
    if kind == "outlier":
        x = rng.standard_normal(K, dtype=np.float32)
        n_out = math.ceil(0.001 * K)
        idx = rng.choice(K, size=n_out, replace=False)
        x[idx] *= np.float32(50.0)
        return x
    raise ValueError(kind)


def _gate_up(rng: np.random.Generator, K: int):
    g = rng.standard_normal(K, dtype=np.float32)
    u = rng.standard_normal(K, dtype=np.float32)
    return g, u


def swiglu_pair(K: int, seed: int):
    """The gate and up rows (float32, N(0,1) each) of one SwiGLU activation."""
    return _gate_up(np.random.default_rng(seed), K)


def swiglu_pairs(w: Workload, nt: int):
    """(g, u) float32 [nt, K] each; column c from its own seed."""
    gu = [swiglu_pair(w.K, act_seed(w, c)) for c in range(nt)]
    return np.stack([a for a, _ in gu]), np.stack([b for _, b in gu])


def activations(w: Workload, nt: int) -> np.ndarray:
    """float32 [nt, K]; column c is drawn from its own seed. Workloads fed by the
    SwiGLU producer draw gate/up pairs instead (swiglu_pairs)."""
    if w.act == "gate_up":
        raise ValueError(f"{w.name}: its activations are gate/up pairs (swiglu_pairs)")
    return np.stack([activation(w.act, w.K, act_seed(w, c)) for c in range(nt)])


def gamma(K: int, seed: int) -> np.ndarray:
    """RMSNorm weight, float32 U[0.5, 1.5]."""
    rng = np.random.default_rng(seed)
    return rng.uniform(0.5, 1.5, size=K).astype(np.float32)


def weights(w: Workload) -> np.ndarray:
    if w.qtype == Q6_K:
        return raw_q6k(w.N, w.K, weight_seed(w))
    return raw_kq(w.qtype, w.N, w.K, weight_seed(w))
