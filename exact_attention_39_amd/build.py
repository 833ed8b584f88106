"""Build libfa.so (the C-ABI attention library) for gfx950 with hipcc.

    python -m exact_attention_39_amd.build        # or build() from Python

Each .hip file under csrc/ is compiled to an object in _build/ (in
parallel), then linked into exact_attention_39_amd/libfa.so in the source
tree, next to the Python binding that loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
POISON_LIB = os.path.join(PKG, "libfa_poison.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_fused.hip"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops (v_pk_add/mul/fma_f32) stay off: the kernels are written for scalar
    # fp32 VALU, and the packed forms are kept out of the generated code as a precaution
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, extra, outdir: str = BUILD) -> str:
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(extra_flags=(), verbose: bool = False) -> str:
    """Compile every kernel source for gfx950 and link libfa.so, and the
    LDS-poison debug build libfa_poison.so (-DFA_LDS_POISON: every direct
    LDS copy first fills its destination with NaN; the GPU tests compare its
    outputs bit for bit with libfa.so).  Always recompiles (this is the
    'does it build' check)."""
    poison_dir = os.path.join(BUILD, "poison")
    os.makedirs(poison_dir, exist_ok=True)
    jobs = [(src, list(extra_flags), BUILD) for src in SOURCES]
    jobs += [(src, list(extra_flags) + ["-DFA_LDS_POISON"], poison_dir) for src in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], POISON_LIB)
    if verbose:
        print(f"built {LIB} and {POISON_LIB}")
    return LIB


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)
