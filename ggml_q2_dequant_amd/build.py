"""Build step for libq2k.so: hipcc for gfx950, in-tree.

Produces ``ggml_q2_dequant_amd/libq2k.so`` (the library behind ``include/q2k.h``)
from the HIP and C++ sources in ``csrc/``, and ``libq2k_probe.so``, the
plain-read measurement kernel the benchmark times beside the path (not part of
the C ABI). Run ``python -m ggml_q2_dequant_amd.build`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libq2k.so")
SOURCES = [os.path.join(CSRC, n) for n in ("q2k_kernels.hip", "q2k_sample.hip", "q2k_moe.hip", "q2k_noalloc.hip",
                                           "q2k_api.cpp", "q2k_gguf.cpp", "q2k_sizes.cpp")]
PROBE_LIB = os.path.join(PKG, "libq2k_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "q2k_probe.hip")]
ARCH = os.environ.get("Q2K_OFFLOAD_ARCH", "gfx950")

# -ffp-contract=off: only FMAs written as such are fused, so every kernel's
# rounding sequence is the one its source spells out. Packed fp32 ops are
# disabled for the device code.
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def _compile(sources, out, verbose: bool) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I" + INCLUDE, "-I" + CSRC, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, "\n".join(msgs)))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile libq2k.so and the measurement library; returns the path of libq2k.so."""
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
