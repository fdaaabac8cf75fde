"""Build libdsa.so for gfx950 with hipcc (objects in parallel, then one link)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")
# measurement kernels of the benchmark's calibration mode, a library of their own
CALIB_LIB = os.path.join(PKG, "libdsa_calib.so")
CALIB_SOURCES = ["calib.hip"]
SOURCES = ["indexer.hip", "topk.hip", "indexer_topk.hip", "sparse_mla.hip", "sparse_mla_bwd.hip", "sparse_mla_bwd_mfma.hip", "indexer_bwd.hip", "indexer_bwd_dense.hip", "prep.hip", "dsa_api.cpp"]
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"),
    # packed fp32 VALU ops off in device code (the host pass warns it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = ["hipcc", *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = ["hipcc", "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(extra: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libdsa.so (and libdsa_calib.so) in the package directory."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES + CALIB_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)
