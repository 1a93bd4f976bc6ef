"""Build libdsa.so (the gfx950 HIP kernels and the C ABI) and libdsa_peaks.so
(the measurement probes) in-tree with hipcc."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
PEAKS_LIB = os.path.join(HERE, "libdsa_peaks.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
SOURCES = ["abi.hip", "indexer.hip", "indexer_fp8.hip", "topk.hip", "sparse_attn.hip",
           "sparse_gqa.hip", "sparse_attn_bwd.hip"]
PEAKS_SOURCES = ["peaks.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay disabled for every gfx950 build
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-I" + INCLUDE,
]


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {PEAKS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
