"""Build libpkv.so (every HIP source under csrc/) for gfx950 with hipcc, and the
benchmark's probe library measure/libpkvceil.so.

Run as `python -m paged_kv_attention_23_amd.build` or through
__graft_entry__.build().  The library lands next to this file.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
ARCH = "gfx950"

# Packed-fp32 VALU instructions are kept out of the generated code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def _compile(src: str, obj: str, save_temps_dir: str | None) -> None:
    cmd = ["hipcc", *HIP_FLAGS, "-c", src, "-o", obj]
    if save_temps_dir:
        cmd.append("-save-temps")
    p = subprocess.run(cmd, capture_output=True, text=True, cwd=save_temps_dir)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr}")
    noise = "is not a recognized feature for this target"
    for line in p.stderr.splitlines():
        if line.strip() and noise not in line:
            print(line, file=sys.stderr)


MEASURE_SRC = os.path.join(HERE, "measure", "ceilings.hip")
MEASURE_LIB = os.path.join(HERE, "measure", "libpkvceil.so")


def build_measure() -> str:
    """The benchmark's reachable-rate probes (plain read, decode-shaped streaming,
    dense matrix loop) as their own small library, outside the attention ABI."""
    tmp = MEASURE_LIB + ".tmp"
    p = subprocess.run(["hipcc", *HIP_FLAGS, "-shared", MEASURE_SRC, "-o", tmp],
                       capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {MEASURE_SRC}:\n{p.stderr}")
    os.replace(tmp, MEASURE_LIB)
    return MEASURE_LIB


def build(save_temps_dir: str | None = None) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    if save_temps_dir:
        os.makedirs(save_temps_dir, exist_ok=True)
        save_temps_dir = os.path.abspath(save_temps_dir)
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], save_temps_dir), zip(srcs, objs)))
    tmp = LIB + ".tmp"
    p = subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, LIB)
    build_measure()
    return LIB


if __name__ == "__main__":
    st = sys.argv[1] if len(sys.argv) > 1 else None
    print(build(st))
