"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

``python -m linear_attention_recurrence_causal_amd.build`` or ``build()``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.hip", "gdn_decode.hip", "gdn_gate.hip", "gdn_prefill.hip", "gdn_prefill_split.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")


def hipcc_cmd(out: str = LIB) -> list[str]:
    return ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU instructions are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}",
            "-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libgdn.so (always recompiles)."""
    tmp = LIB + ".tmp"
    r = subprocess.run(hipcc_cmd(tmp), capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
