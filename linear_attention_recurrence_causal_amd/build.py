"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

``python -m linear_attention_recurrence_causal_amd.build`` or ``build()``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn.so")
SOURCES = ["gdn_api.hip", "gdn_decode.hip", "gdn_gate.hip", "gdn_prefill.hip", "gdn_prefill_split.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")


FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 VALU instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libgdn.so (always recompiles): one hipcc
    per source in parallel, then the link."""
    from concurrent.futures import ThreadPoolExecutor
    tmpdir = tempfile.mkdtemp(prefix="gdn_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        jobs = [["hipcc"] + FLAGS + ["-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
            errs = list(ex.map(_run, jobs))
        tmp = LIB + ".tmp"
        errs.append(_run(["hipcc", f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", tmp] + objs))
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    err = "\n".join(e for e in errs if e.strip())
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


DEMO_SRC = os.path.join(ROOT, "tests", "c_abi", "gdn_c_demo.cpp")
DEMO_BIN = os.path.join(ROOT, "tests", "c_abi", "gdn_c_demo")


def build_c_demo(verbose: bool = False) -> str:
    """The C-ABI caller of tests/c_abi (host code, linked against libgdn.so)."""
    tmp = DEMO_BIN + ".tmp"
    err = _run(["hipcc", "-O2", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", "-o", tmp, DEMO_SRC,
                f"-L{PKG}", "-lgdn", "-Wl,-rpath,$ORIGIN/../../linear_attention_recurrence_causal_amd"])
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, DEMO_BIN)
    return DEMO_BIN


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_demo(verbose=True))
