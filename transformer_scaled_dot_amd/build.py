"""Build the HIP library in-tree: transformer_scaled_dot_amd/libattn_fwd.so (gfx950 only).

    python -m transformer_scaled_dot_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn_fwd.so")
SOURCES = ["attn_fwd_api.hip", "attn_fwd_mfma.hip", "attn_fwd_f32.hip", "attn_merge.hip",
           "attn_bwd_api.hip", "attn_bwd_mfma.hip", "attn_bwd_f32.hip"]
HEADERS = ["attn_common.h", "attn_bwd.h", os.path.join(ROOT, "include", "attn_fwd.h"),
           os.path.join(ROOT, "include", "attn_bwd.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # packed fp32 arithmetic stays off: the compiler would otherwise form v_pk_* fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
