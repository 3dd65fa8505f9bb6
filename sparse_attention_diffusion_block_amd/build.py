"""Compile librettn.so (the C ABI of include/rettn.h) for gfx950 with hipcc.

Each HIP source is compiled to an object in parallel, then linked into a
shared library that sits next to this file, where the binding loads it.
The issue-cost and HBM streaming probes (standalone measurement programs, not
part of the library) are built beside it as `probe_issue` and `probe_stream`.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librettn.so")
PROBES = [os.path.join(HERE, "probe_issue"), os.path.join(HERE, "probe_stream")]
SOURCES = ["host.cpp", "abi.hip", "attn_bf16.hip", "attn_f32.hip", "index.hip", "sparse64.hip", "calib.hip", "dynamic.hip", "sparse_wg.hip"]
ARCH = "gfx950"
# Packed fp32 instructions are disabled in all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False):
    """Compile every HIP source and link librettn.so; always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [[hipcc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    for probe in PROBES:
        cmds.append([hipcc, *FLAGS, os.path.join(CSRC, os.path.basename(probe) + ".hip"), "-o", probe + ".tmp"])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    _check_launch_stubs(tmp)
    os.replace(tmp, LIB)
    for probe in PROBES:
        os.replace(probe + ".tmp", probe)
    return LIB


def _check_launch_stubs(path):
    """Fail the build if a kernel's host launch stub is missing.  The host pass of hipcc has been
    seen to skip emitting a stub, for some arrangements of lambdas and arrays in a kernel body,
    without any diagnostic; the library then links and only fails when it is loaded."""
    nm = shutil.which("nm") or "/opt/rocm/llvm/bin/llvm-nm"
    p = subprocess.run([nm, "-D", "--undefined-only", path], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    missing = [l.split()[-1] for l in p.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError(f"{path}: kernel launch stubs missing from the host code: {missing[:4]}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
