"""Build libfavor.so in-tree with hipcc for gfx950.

    python -m efficient_transformer_attention_favor_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("favor_kernels.hip", "favor_features.hip", "favor_decode.hip",
                                                  "favor_backward.hip", "favor_draw.hip", "favor_generalized.hip", "favor_causal.hip", "favor_small.hip",
                                                  "favor_plan.cpp")]
OUTPUT = os.path.join(PKG, "libfavor.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    tmp = OUTPUT + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
