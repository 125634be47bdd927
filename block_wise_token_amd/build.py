"""Build libuniprefill.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m block_wise_token_amd.build   (or call build())
Object files go to <repo>/_build/, the library to block_wise_token_amd/libuniprefill.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libuniprefill.so")
# The GEMMs of the layer on the survivors (hipBLASLt) live in a library of their own.
LAYER_LIB = os.path.join(PKG, "libuniprefill_layer.so")
SOURCES = ["abi.hip", "score.hip", "select.hip", "compact.hip", "consumer.hip"]
LAYER_SOURCES = ["gemm.hip"]
# A measurement program (not linked into either library): the sustained clock and matrix
# rate of the score kernel's instruction mix.
PROBE_SRC = "probe_mfma_mix.hip"
PROBE_BIN = os.path.join(PKG, "probe_mfma_mix")
ARCH = "gfx950"

# Packed-FP32 instructions are switched off for all device code.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libuniprefill")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(noise))
    if any(ln.strip() for ln in noise):
        print("\n".join(noise), file=sys.stderr)
    return obj


def _link(objs, out, extra, shared=True):
    tmp = out + ".tmp"
    kind = ["-shared", "-fPIC"] if shared else []
    cmd = [hipcc(), *kind, f"--offload-arch={ARCH}", *objs, *extra, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + LAYER_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    # The decision library: HIP runtime only.
    _link([objs[s] for s in SOURCES], LIB, ["-Wl,-soname,libuniprefill.so"])
    # The layer's GEMMs: hipBLASLt, and libuniprefill.so (found next to it) for the gate.
    _link([objs[s] for s in LAYER_SOURCES], LAYER_LIB,
          ["-L", PKG, "-luniprefill", "-lhipblaslt", "-Wl,-rpath,$ORIGIN",
           "-Wl,-soname,libuniprefill_layer.so"])
    _link([_compile(PROBE_SRC)], PROBE_BIN, [], shared=False)
    if verbose:
        print(f"built {LIB}, {LAYER_LIB} and {PROBE_BIN}")
    return LIB


if __name__ == "__main__":
    build()
