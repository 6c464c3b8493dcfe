"""Build libsgmv.so in-tree for gfx950 with hipcc.

HIP sources are compiled by hipcc for gfx950 (packed fp32 instructions disabled), the
host-only segment builder by g++; the objects are linked by hipcc into
``segmented_gather_gemv_amd/libsgmv.so``. The benchmark's streaming reference kernel
(``csrc/bench/``, not part of the library) goes into ``libsgmv_bench.so``, and a profiling copy
of the library whose single-launch kernel records phase stamps (``-DSGMV_PHASE_STAMPS``) into
``libsgmv_stamps.so``. Always rebuilds. Run as
``python -m segmented_gather_gemv_amd.build`` or call ``build()``.
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
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsgmv.so")
BENCH_LIB = os.path.join(PKG, "libsgmv_bench.so")
STAMPS_LIB = os.path.join(PKG, "libsgmv_stamps.so")
STAMPED = "delta_bf16_build.hip"  # the source compiled again with the stamps
BENCH_SRC = os.path.join(CSRC, "bench")
ARCH = os.environ.get("SGMV_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libsgmv")
    return p


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(f for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    hipcc = _hipcc()
    hip, cpp = sources()
    cmds = []
    objs = []
    for f in hip:
        o = os.path.join(OUT_DIR, f + ".o")
        objs.append(o)
        cmds.append([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
    for f in cpp:
        o = os.path.join(OUT_DIR, f + ".o")
        objs.append(o)
        cmds.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, f), "-o", o])
    stamp_obj = os.path.join(OUT_DIR, "stamps_" + STAMPED + ".o")
    cmds.append([hipcc, *HIP_FLAGS, "-DSGMV_PHASE_STAMPS", "-c", os.path.join(CSRC, STAMPED),
                 "-o", stamp_obj])
    bench_objs = []
    for f in sorted(f for f in os.listdir(BENCH_SRC) if f.endswith(".hip")):
        o = os.path.join(OUT_DIR, "bench_" + f + ".o")
        bench_objs.append(o)
        cmds.append([hipcc, *HIP_FLAGS, "-c", os.path.join(BENCH_SRC, f), "-o", o])
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = STAMPS_LIB + ".tmp"
    stamp_objs = [o for o in objs if os.path.basename(o) != STAMPED + ".o"] + [stamp_obj]
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *stamp_objs])
    os.replace(tmp, STAMPS_LIB)
    tmp = BENCH_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *bench_objs])
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
