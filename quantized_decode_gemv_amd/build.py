"""Build libq6kdpl.so (HIP, gfx950) in-tree with hipcc.

    python -m quantized_decode_gemv_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libq6kdpl.so")
SOURCES = ["abi.hip", "mmvq.hip", "producer.hip", "repack.hip", "tiles.hip"]
# the read-bandwidth probe of the measurement harness (bench.py --read-ceiling), a
# library of its own so the GEMV library holds only the path
PROBE_LIB = os.path.join(PKG, "libq6kprobe.so")
PROBE_SOURCES = ["read_probe.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instruction forms (v_pk_*_f32) in any device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no implicit multiply-add contraction: every fused multiply-add is written out,
    # so kernels that share arithmetic round identically
    "-ffp-contract=off",
    # matrix-core instructions accumulate in ordinary vector registers: their results
    # feed vector arithmetic at once, and the accumulation-register form adds one copy
    # per result register
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def _hipcc(srcs, out: str, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Builds the GEMV library and the measurement probe; returns the library path."""
    _hipcc([os.path.join(CSRC, s) for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return _hipcc(sources(), LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
