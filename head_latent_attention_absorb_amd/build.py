"""Build the gfx950 HIP library ``libmla_absorb.so`` in-tree with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(REPO_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libmla_absorb.so")

SOURCES = ["abi.hip", "absorb_out.hip", "append.hip", "quant.hip", "combine_out.hip", "decode_generic.hip", "decode_mfma.hip", "prefill.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 VALU ops are kept out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    "-I" + os.path.join(REPO_DIR, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(line for line in r.stderr.splitlines()
                     if "packed-fp32-ops" not in line and line.strip())
    if warn.strip():
        print(f"[build] {src}:\n{warn}", file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link ``libmla_absorb.so``.

    Always recompiles.  Returns the library path.
    """
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"[build] wrote {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
