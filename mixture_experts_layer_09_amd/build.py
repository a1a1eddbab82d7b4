"""Build the HIP library (libmoe.so) and the host-only planner (libmoe_plan.so).

    python mixture_experts_layer_09_amd/build.py

libmoe.so     : every .hip source plus the planner, hipcc for gfx950 only.
libmoe_plan.so: the planner/validator alone, built with g++ (no HIP), so that
                the argument checks can be exercised on a machine with no GPU.
Both land next to this file (in-tree) and are loaded from there.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
PLAN_LIB = os.path.join(HERE, "libmoe_plan.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 arithmetic stays off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + out)
    return out


def sources():
    hip = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    return [os.path.join(CSRC, f) for f in hip] + [os.path.join(CSRC, "moe_plan.cpp")]


def build_plan_lib(cxx="g++"):
    _run([cxx, "-std=c++17", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
          os.path.join(CSRC, "moe_plan.cpp"), "-o", PLAN_LIB + ".tmp"])
    os.replace(PLAN_LIB + ".tmp", PLAN_LIB)
    return PLAN_LIB


def build_hip_lib(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()

    def obj(src):
        o = os.path.join(BUILD, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        out = _run([HIPCC] + HIP_FLAGS + lang + ["-c", src, "-o", o])
        if verbose and out.strip():
            print(out)
        return o

    n = jobs or min(8, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(n) as ex:
        objs = list(ex.map(obj, srcs))
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", LIB + ".tmp"])
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build(verbose=False):
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    build_plan_lib()
    return build_hip_lib(verbose=verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
