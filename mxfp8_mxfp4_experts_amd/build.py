"""Build ``libmi355moe.so`` (gfx950) in-tree with hipcc.

Run ``python -m mxfp8_mxfp4_experts_amd.build`` or call ``build()``.  Every
source is compiled on each call (a cross-compile: no GPU is needed).
``build_rates()`` builds the benchmark's rate probes
(``measure/libmi355rates.so``) and ``build_probes()`` the test-only probe
library (``tests/probe/libnumprobe.so``); neither is part of the layer.
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
OUT = os.path.join(PKG, "libmi355moe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Wno-unused-value",
    # Leave packed FP32 instructions to no code path (a known hazard on these parts).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out


def _build_so(sources, out_path, tag, verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, tag + "_" + os.path.basename(src) + ".o")
        rc, out = _run([HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj])
        return src, obj, rc, out

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(compile_one, sources))
    failed = False
    for src, obj, rc, out in results:
        if out.strip() and (verbose or rc != 0):
            print(f"[build] {os.path.basename(src)}:\n{out}", file=sys.stderr)
        if rc != 0:
            failed = True
        objs.append(obj)
    if failed:
        raise RuntimeError("hipcc failed; see messages above")
    tmp = out_path + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    if rc != 0:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, out_path)
    if verbose:
        print(f"[build] wrote {out_path}")
    return out_path


def build(verbose: bool = False, jobs: int = 8) -> str:
    """The layer library ``libmi355moe.so`` from every source in csrc/."""
    return _build_so(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), OUT, "lib", verbose, jobs)


MEASURE_DIR = os.path.join(PKG, "measure")
MEASURE_OUT = os.path.join(MEASURE_DIR, "libmi355rates.so")


def build_rates(verbose: bool = False) -> str:
    """The benchmark's achievable-rate probes (streaming HBM read, scaled
    MFMA loop); not part of the layer library."""
    return _build_so([os.path.join(MEASURE_DIR, "rates.hip")], MEASURE_OUT, "rates", verbose)


PROBE_DIR = os.path.join(ROOT, "tests", "probe")
PROBE_OUT = os.path.join(PROBE_DIR, "libnumprobe.so")


def build_probes(verbose: bool = False) -> str:
    """The test-only probe library (device functions of the FC kernels run
    on inputs the GPU tests choose)."""
    return _build_so([os.path.join(PROBE_DIR, "numerics_probe.hip")], PROBE_OUT, "probe",
                     verbose)


if __name__ == "__main__":
    build(verbose=True)
    build_rates(verbose=True)
    build_probes(verbose=True)
