"""Python binding of libq6kdpl.so, the q6_K x q8 decode GEMV for MI355X (gfx950).

Argument marshalling only: every entry point forwards to the C ABI declared in
include/q6kdpl.h with the same name. Device buffers are torch tensors (or raw
integer device pointers); the stream defaults to torch's current stream. Every
step of the path runs in the HIP kernels; there is no CPU fallback, and a
missing or unloadable library raises.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    KQ_Q4_K, KQ_Q5_K, KQ_Q6_K, LIB_PATH, Q6K_MAX_K, Q6K_MAX_N, Q6K_MAX_NT, Q6kError,
    gate_up_swiglu_fused, kq_block_bytes, kq_dpl_bytes, kq_dpl_row_stride, kq_raw_bytes, lib,
    load, mmvq_kq_gate_up_swiglu_q8, mmvq_kq_q8,
    mmvq_kq_q8_subdots, mmvq_kq_rmsnorm_q8, mmvq_plan, repack_kq_dpl, repack_kq_dpl_host,
    unpack_kq_dpl_host,
    mmvq_q6k_q8, mmvq_q6k_q8_subdots, mmvq_q6k_rmsnorm_q8, q6k_dpl_bytes, q6k_dpl_row_stride, q6k_raw_bytes,
    q6k_version, q8_plane_bytes, quant_q8, repack_q6k_dpl, repack_q6k_dpl_host,
    rmsnorm_mmvq_fused, rmsnorm_quant_q8, swiglu_quant_q8, unpack_q6k_dpl_host,
)
