"""Build libduo_attn.so in-tree with hipcc for gfx950.

    python -m mixed_head_kv_amd.build          # compile every source, link the library

It also builds libduo_inputs.so, the host (C, OpenMP) twin of the seeded input
generator that the tests and the bench's CPU baseline use for long histories.

Every HIP source compiles with packed-fp32 instructions disabled and with correctly
rounded fp32 division (the int4 quantiser's divisions must round like the format's
definition).  Objects go to mixed_head_kv_amd/_build/, the library next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libduo_attn.so")
ARCH = "gfx950"

SOURCES = ["duo_attn.cpp", "kv_cache.hip", "attention_valu.hip"]
EXTRA_SOURCES = ["decode_mfma.hip", "prefill_mfma.hip", "linear_w8.hip"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math", "-Wall", "-Wno-unused-function",
]


# Per-source additions.  The pre-filling kernel computes with finite values or -inf only
# (scores, running maxima, weights), so it builds without NaN semantics: its maxima then
# need no quieting of their inputs (5 fewer VALU instructions per 64-key tile).
FILE_FLAGS = {
    "prefill_mfma.hip": ["-fno-honor-nans"],
}


def flags_for(src: str) -> list:
    """hipcc flags for one source file."""
    return HIP_FLAGS + FILE_FLAGS.get(src, [])


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return p


def sources():
    out = list(SOURCES)
    for s in EXTRA_SOURCES:
        if os.path.exists(os.path.join(CSRC, s)):
            out.append(s)
    return out


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags_for(src), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


INPUTS_SRC = os.path.join(HERE, "inputs_host.c")
INPUTS_LIB = os.path.join(HERE, "libduo_inputs.so")


def build_inputs(verbose: bool = False) -> str:
    """The host twin of the seeded input generator (plain C, gcc with OpenMP)."""
    tmp = INPUTS_LIB + ".tmp"
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", INPUTS_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed for inputs_host.c:\n" + r.stdout + r.stderr)
    os.replace(tmp, INPUTS_LIB)
    return INPUTS_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    build_inputs(verbose)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
