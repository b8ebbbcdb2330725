"""Build libla.so, the gfx950 HIP library behind include/la.h.

    python -m gated_delta_rule_causal_amd.build [-j N]

Each source under csrc/ is compiled by hipcc for gfx950 into _build/, then
linked into gated_delta_rule_causal_amd/libla.so (in-tree, next to the
binding that loads it).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "la")
LIB = os.path.join(PKG, "libla.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-I" + INCLUDE, "-I" + CSRC,
    # no packed-fp32 (v_pk_*_f32) instructions anywhere in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

SOURCES = ["la_api.cpp", "la_decode.hip", "la_chunk_linear.hip", "la_chunk_segment.hip", "la_chunk_gdr.hip",
           "la_chunk_kda.hip", "la_chunk_bwd.hip"]
# peak probes (a streaming copy, a matrix-core loop), a library of their own
PROBE_SOURCES = ["la_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libla_probe.so")


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC] + COMMON_FLAGS + ["-x", "hip", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libla.so; returns its path."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found (set HIPCC)")
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES) + len(PROBE_SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, lib)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-j", "--jobs", type=int, default=None)
    args = ap.parse_args(argv)
    build(jobs=args.jobs, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
