"""Build libla.so for gfx950 in-tree with hipcc.

    python -m non_causal_linear_amd.build

csrc/la_kernels.hip is compiled once per (element type, Q/K head size) unit,
the units in parallel, and linked with csrc/la_api.cpp and csrc/la_scratch.hip
(the static device scratch of la_fwd_noalloc) into
non_causal_linear_amd/libla.so (written to a temporary name and renamed, so
a process that has the old library open keeps a consistent file).
"""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libla.so")
# what built LIB (compiler version and flags), written beside it; bench.py reports it
BUILD_INFO = os.path.join(PKG, "libla.build.json")

KERNELS = "la_kernels.hip"
API = "la_api.cpp"
SCRATCH = "la_scratch.hip"
# (la_dtype, DK) of every kernel unit; each covers all DV (DK = 256: 16-bit, DV = 256)
UNITS = [(dt, dk) for dt in (0, 1, 2) for dk in (32, 64, 96, 128)] + [(1, 256), (2, 256)]

# Packed fp32 VALU forms are switched off for every HIP source.
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# A unit instantiates one element type: the helpers written for the others
# (16-bit MFMA wrappers, the f16 scaling) are unused there.
UNIT_FLAGS = ["-Wno-unused-function", "-Wno-unused-const-variable", "-Wno-unneeded-internal-declaration"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is expected under /opt/rocm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res.stderr


def build(verbose: bool = False, jobs: int | None = None) -> str:
    cc = hipcc()
    inc = ["-I", INCLUDE, "-I", CSRC]
    jobs = jobs or min(len(UNITS), max(1, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory(prefix="la_build_") as tmpdir:
        objs, cmds = [], []
        for dt, dk in UNITS:
            obj = os.path.join(tmpdir, f"la_kernels_{dt}_{dk}.o")
            objs.append(obj)
            cmds.append([cc, *HIPCC_FLAGS, *UNIT_FLAGS, *inc, f"-DLA_UNIT_DTYPE={dt}", f"-DLA_UNIT_DK={dk}",
                         "-c", os.path.join(CSRC, KERNELS), "-o", obj])
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            warnings = list(pool.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp%d" % os.getpid()
        try:
            warnings.append(_run([cc, *HIPCC_FLAGS, "-shared", *inc, *objs, os.path.join(CSRC, API),
                                  os.path.join(CSRC, SCRATCH), "-o", tmp], verbose))
        except Exception:
            if os.path.exists(tmp):
                os.unlink(tmp)
            raise
    if verbose:
        text = "".join(w for w in warnings if w.strip())
        if text:
            print(text, file=sys.stderr)
    os.replace(tmp, LIB)
    ver = subprocess.run([cc, "--version"], capture_output=True, text=True).stdout
    info = {"hipcc": next((ln.strip() for ln in ver.splitlines() if "HIP version" in ln), None),
            "flags": HIPCC_FLAGS, "units": [list(u) for u in UNITS]}
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
