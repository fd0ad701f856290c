"""Compile libgdnbeam.so for gfx950 in-tree with hipcc.

Every kernel source is compiled to an object in ``_build/`` (in parallel),
then linked into ``linear_attention_beam_gdn_amd/libgdnbeam.so``.  Two
measurement libraries are built beside it: ``libgdnbeam_stamps.so``, the same
library with the fused kernels' clock stamps compiled in (GDN_STAMPS),
``libgdnbeam_check.so``, the library with device-side parent-pointer checks
(GDN_CHECK_PARENTS, include/gdn_beam_check.h), and
``measure/libgdnmeasure.so``, the streaming-rate reference kernels.  All HIP
code is built with packed-FP32 instructions disabled.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdnbeam.so")
STAMPS_LIB = os.path.join(PKG, "libgdnbeam_stamps.so")
MEASURE_SRC = os.path.join(PKG, "measure", "k_stream.hip")
MEASURE_LIB = os.path.join(PKG, "measure", "libgdnmeasure.so")
STAMPED = ("k_beam_fused.hip", "k_beam_fused_kda.hip")  # the sources built a second time with GDN_STAMPS
CHECK_LIB = os.path.join(PKG, "libgdnbeam_check.so")
# the sources that read parent pointers (or own the counter), built again with GDN_CHECK_PARENTS
CHECKED = ("abi.hip", "k_beam_decode.hip", "k_beam_fused.hip", "k_beam_fused_kda.hip")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def _compile(src: str, extra=(), suffix="") -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", suffix + ".o"))
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    stamped = [os.path.join(CSRC, f) for f in STAMPED]
    checked = [os.path.join(CSRC, f) for f in CHECKED]
    jobs = [(s, tuple(extra), "") for s in srcs]
    jobs += [(st, tuple(extra) + ("-DGDN_STAMPS",), "_stamps") for st in stamped]
    jobs += [(c, tuple(extra) + ("-DGDN_CHECK_PARENTS",), "_check") for c in checked]
    jobs.append((MEASURE_SRC, tuple(extra), ""))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    n, ns, nc = len(srcs), len(stamped), len(checked)
    prod = objs[:n]
    _link(prod, LIB)
    _link([o for o, s in zip(prod, srcs) if s not in stamped] + objs[n:n + ns], STAMPS_LIB)
    _link([o for o, s in zip(prod, srcs) if s not in checked] + objs[n + ns:n + ns + nc], CHECK_LIB)
    _link([objs[-1]], MEASURE_LIB)
    if verbose:
        print(f"built {LIB} (and {os.path.basename(STAMPS_LIB)}, {os.path.basename(CHECK_LIB)}, "
              f"measure/{os.path.basename(MEASURE_LIB)})")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
