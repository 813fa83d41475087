"""Build libslora.so (HIP, gfx950) in-tree.

Host sources (.cpp) are compiled as plain C++ against the HIP runtime headers;
kernel sources (.hip) with hipcc for gfx950 only. Packed fp32 instructions are
disabled in device code (-packed-fp32-ops); all device arithmetic is scalar fp32,
fp16/bf16 dot2 and MFMA.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libslora.so")
BUILD_DIR = os.path.join(ROOT, "_build", "slora")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HOST_SRCS = ["pool.cpp", "plan.cpp", "api.cpp", "sched.cpp"]
DEVICE_SRCS = ["mbgmv.hip", "sgmv.hip", "fetch.hip", "noalloc.hip", "gather.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"-I{CSRC}", "-D__HIP_PLATFORM_AMD__=1"]


def _cmd_host(src, obj):
    return [os.path.join(ROCM, "llvm", "bin", "clang++"), *COMMON, f"-I{ROCM}/include",
            "-c", src, "-o", obj]


def _cmd_device(src, obj):
    return [os.path.join(ROCM, "bin", "hipcc"), "-x", "hip", f"--offload-arch={ARCH}", *COMMON,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-c", src, "-o", obj]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in p.stderr.splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the device feature
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tasks = []
    for s in HOST_SRCS:
        tasks.append(_cmd_host(os.path.join(CSRC, s), os.path.join(BUILD_DIR, s + ".o")))
    for s in DEVICE_SRCS:
        tasks.append(_cmd_device(os.path.join(CSRC, s), os.path.join(BUILD_DIR, s + ".o")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for msg in ex.map(_run, tasks):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    objs = [t[-1] for t in tasks]
    tmp = OUT + ".tmp"
    _run([os.path.join(ROCM, "bin", "hipcc"), f"--offload-arch={ARCH}", "-shared", "-fPIC",
          "-o", tmp, *objs, f"-L{ROCM}/lib", "-lamdhip64", "-Wl,-rpath," + f"{ROCM}/lib"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
