"""Build the gfx950 shared library ``libsemicrf.so`` in-tree with hipcc.

Every call compiles all sources again (object files go to ``_build/``), then links
``semi_markov_crf_amd/libsemicrf.so`` and the peak-rate microbenchmark
``libsemicrf_peak.so`` that bench.py uses.  Usage: ``python -m semi_markov_crf_amd.build``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsemicrf.so")
# the peak-rate microbenchmark behind bench.py's roofline, a library of its own
PEAK_LIB = os.path.join(HERE, "libsemicrf_peak.so")
PEAK_SOURCES = ["peak.hip"]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_*_f32 in generated code.  -fno-honor-nans: fmax without the
# NaN-quieting canonicalisation (inputs are finite or -inf by contract).  Range checks
# combine booleans bitwise on purpose (no short-circuit branches).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-honor-nans",
    "-Wall", "-Wno-unused-result", "-Wno-bitwise-instead-of-logical",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]

SOURCES = ["api.cpp", "sweep_cfg.cpp", "scan.hip", "sweep_lse_mirror.hip", "sweep_lse_plain.hip",
           "sweep_lse_log.hip", "sweep_maxplus_mirror.hip", "sweep_maxplus_plain.hip",
           "sweep_round_proj.hip", "sweep_round_proj_log.hip", "marginals.hip", "gold.hip", "viterbi.hip", "seam.hip",
           "sweep_xk_lse.hip", "sweep_xk_maxplus.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PEAK_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PEAK_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PEAK_LIB)
    if verbose:
        print(f"built {LIB} and {PEAK_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
