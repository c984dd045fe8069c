"""Build the gfx950 shared library ``libsparse_attn.so`` in-tree with hipcc.

    python -m sparse_attention_long_page_amd.build        # build (always recompiles)

Every source under csrc/ is compiled for gfx950 only; the objects are linked
into one shared library next to this file, which the Python binding loads.
Packed fp32 instructions are disabled for device code
(-target-feature -packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsparse_attn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "summary_score.hip", "select.hip", "decode.hip", "mla.hip", "prefill.hip",
           "select_decode.hip", "validate.hip", "mask.hip", "meancorr.hip", "autotune.hip"]

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") or src.endswith(".cpp") else []
    cmd = [hipcc()] + lang + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{msgs}")
    if msgs:
        sys.stderr.write(msgs + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    # a kernel template whose host-side instantiation failed leaves its launch
    # stub undefined, which would only show when the library is loaded: fail here
    nm = shutil.which("nm")
    if nm:
        r = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True)
        missing = [l.split()[-1] for l in r.stdout.splitlines() if l.split() and l.split()[-1].startswith("_ZN2sa")]
        if missing:
            os.remove(tmp)
            raise RuntimeError(f"undefined library symbols after linking: {missing}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
