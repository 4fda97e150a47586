"""Builds the HIP library of the MoE expert layer in-tree for gfx950.

Each ``csrc/*.hip`` is compiled to an object under ``_build/`` (in parallel), then
linked into ``moe_expert_layer_amd/libmoe_expert_layer.so``.  The measurement probes
(``probes/*.hip``, not part of the layer) are linked into ``libmoe_probes.so`` beside it.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_expert_layer.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
PROBE_DIR = os.path.join(PKG, "probes")
PROBE_LIB_PATH = os.path.join(PKG, "libmoe_probes.so")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 math is disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return p


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, path: str):
    tmp = path + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, path)


def build(extra_flags=(), verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the layer library and the probe library;
    returns the layer library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    psrcs = sorted(glob.glob(os.path.join(PROBE_DIR, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), srcs + psrcs))
    _link(objs[:len(srcs)], LIB_PATH)
    _link(objs[len(srcs):], PROBE_LIB_PATH)
    if verbose:
        print("built", LIB_PATH, "and", PROBE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
