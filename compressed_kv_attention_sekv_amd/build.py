"""Compile the SeKV HIP library for gfx950: one shared object, libsekv.so,
next to this file.  Run ``python -m compressed_kv_attention_sekv_amd.build``.

``--timeline`` builds a diagnostic copy instead, libsekv_timeline.so, whose
route, attend and tail workgroups record time stamps (SEKV_TIMELINE in
sekv_decode.hip); load it with SEKV_LIBRARY for ``bench.py --timeline``."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsekv.so")
OUT_TIMELINE = os.path.join(HERE, "libsekv_timeline.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["sekv_api.cpp", "sekv_build.hip", "sekv_decode.hip", "sekv_cap.hip",
           "sekv_resident.hip", "sekv_gates.hip", "sekv_rsvd.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # packed fp32 instructions stay off (hipcc's host pass warns it does not know the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-result",
]


def _jobs() -> int:
    n = os.environ.get("MAX_JOBS")
    return max(1, min(len(SOURCES), int(n) if n and n.isdigit() else (os.cpu_count() or 1)))


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compile every source (in parallel, one hipcc per file) and link; with
    `timeline`, the time-stamped diagnostic library."""
    from concurrent.futures import ThreadPoolExecutor
    bdir = os.path.join(BUILD_DIR, "timeline") if timeline else BUILD_DIR
    out = OUT_TIMELINE if timeline else OUT
    flags = FLAGS + (["-DSEKV_TIMELINE"] if timeline else [])
    os.makedirs(bdir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmds.append([HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)

    def compile_one(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for f in [ex.submit(compile_one, c) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv))
