"""Build the gfx950 HIP library ``libgqa_hip.so`` in-tree with hipcc.

Usage: ``python -m grouped_query_attention_03_amd.build`` (or ``build()``).
Every call recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libgqa_hip.so")
SOURCES = ["gqa_api.hip", "prefill_bf16.hip", "prefill_f32.hip", "decode_bf16.hip",
           "rope_bf16.hip"]
# Select the VGPR form of MFMA instructions: the register allocator then moves
# only accumulator chains that never feed vector ALU work to AGPRs.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
# The bf16 prefill kernel never orders NaNs (masked and stale scores are
# replaced by -inf with a select before any max), so it runs with the IEEE
# mode bit off: max/min then need no canonicalising copies.
NO_IEEE = ["-fno-honor-nans", "-mno-amdgpu-ieee"]
# Per-source flags (default: VGPR_FORM).
SOURCE_FLAGS = {"prefill_bf16.hip": VGPR_FORM + NO_IEEE}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# hipcc's host pass does not know the packed-fp32 feature; that note is harmless
_NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if _NOISE not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every HIP source into ``libgqa_hip.so`` (always recompiles)."""
    tag = ".tmp%d" % os.getpid()
    objs = []
    try:
        for src in SOURCES:
            obj = os.path.join(PKG_DIR, src + tag + ".o")
            objs.append(obj)
            _run([HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, VGPR_FORM), *extra_flags, "-I", INCLUDE,
                  "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        tmp = LIB_PATH + tag
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB_PATH)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True, extra_flags=sys.argv[1:]))
