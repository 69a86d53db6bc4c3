"""Build libcsa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_attention_decode_csa_amd.build

Each .hip source is compiled to an object in parallel, then linked into
sparse_attention_decode_csa_amd/libcsa.so next to this file.  The memory
ceiling probes (csrc/ceilings.hip, include/csa_ceilings.h) are linked into a
library of their own, libcsa_ceilings.so, which the decode path never loads.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcsa.so")
CEILINGS_LIB = os.path.join(PKG, "libcsa_ceilings.so")
CEILINGS_SOURCES = ["ceilings.hip"]
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "indexer_score.hip", "topk.hip", "sparse_attn.hip", "swa_writeback.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str, obj_dir: str = OBJ_DIR, defines=()) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile and link; `defines` override tuning constants (e.g. for sweeps).
    The default build also links the ceiling probes' library."""
    obj_dir = OBJ_DIR if out == LIB else out + ".objs"
    os.makedirs(obj_dir, exist_ok=True)
    _link(SOURCES, out, obj_dir, defines, verbose)
    if out == LIB:
        _link(CEILINGS_SOURCES, CEILINGS_LIB, obj_dir, (), verbose)
    return out


def _link(sources, out: str, obj_dir: str, defines, verbose: bool) -> None:
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(sources)) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, defines), sources))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # A shared library links with undefined symbols; every symbol of the
    # library's own namespace must be defined inside it (a missing kernel
    # stub would otherwise surface only when the library is loaded).
    r = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if "_ZN3csa" in ln]
    if r.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError(f"{out}: undefined library symbols {missing[:4]} ({len(missing)})")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
