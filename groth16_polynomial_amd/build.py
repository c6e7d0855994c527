"""Builds libg16.so (the HIP library) and libg16_probe.so (the instruction-rate probe the
benchmark uses for its roofline) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libg16.so")
PROBE_LIB = os.path.join(PKG, "libg16_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed FP32 instructions stay disabled (none of this code is floating point)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]

# The narrow-geometry units (small launches, each thread's chain of dependent products
# sets the time) are scheduled for instruction-level parallelism.
UNIT_FLAGS = {"_narrow.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def unit_flags(unit: str) -> list:
    return [f for suffix, fl in UNIT_FLAGS.items() if unit.endswith(suffix) for f in fl]


def sources() -> list:
    csrc = os.path.join(PKG, "csrc")
    return sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                  if f.endswith((".hip", ".hpp", ".h")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every translation unit (always recompiles) in parallel, link, and return
    the library path.  The probe library is built alongside."""
    csrc = os.path.join(PKG, "csrc")
    units = sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = jobs or min(len(units) + 1, int(os.environ.get("MAX_JOBS", "8")), os.cpu_count() or 1)
    objs = []
    cmds = []
    for u in units:
        obj = os.path.join(objdir, u.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *compile_flags, *unit_flags(u), *inc, "-c", "-o", obj,
                     os.path.join(csrc, u)])
    probe_tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmds.append([HIPCC, *FLAGS, "-o", probe_tmp, os.path.join(csrc, "probe", "mad_rate.hip")])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    os.replace(probe_tmp, PROBE_LIB)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
