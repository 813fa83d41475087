"""The library's host-only logic (page pool, planner, residency manager, admission
scheduler, argument validation) under AddressSanitizer and UndefinedBehaviorSanitizer.

The host sources are compiled here with the sanitizers (plain clang++, host code only;
the kernel objects are the normal build's, linked unchanged), together with the
randomized driver in tests/host_sanitize/driver.cpp, which checks the invariants it can
see as it goes. No GPU is used."""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CXX = os.path.join(ROCM, "llvm", "bin", "clang++")
HOST_SRCS = ["pool.cpp", "plan.cpp", "api.cpp", "sched.cpp"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, **kw)
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    assert p.returncode == 0, f"{' '.join(cmd)}\n{err}\n{p.stdout}"
    return p


@pytest.mark.skipif(not os.path.exists(CXX), reason="ROCm clang++ not found")
def test_host_logic_under_sanitizers(tmp_path):
    from heterogeneous_lora_amd import build
    csrc = os.path.join(ROOT, "heterogeneous_lora_amd", "csrc")
    dev_objs = [os.path.join(build.BUILD_DIR, s + ".o") for s in build.DEVICE_SRCS]
    if not all(os.path.exists(o) for o in dev_objs):
        build.build()
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}", f"-I{ROCM}/include",
           "-D__HIP_PLATFORM_AMD__=1"]
    objs = []
    for s in HOST_SRCS + ["driver.cpp"]:
        src = os.path.join(csrc, s) if s != "driver.cpp" else \
            os.path.join(ROOT, "tests", "host_sanitize", s)
        obj = str(tmp_path / (s + ".o"))
        _run([CXX, "-O1", "-g", "-std=c++17", *SAN, *inc, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "host_driver")
    _run([CXX, *SAN, "-o", exe, *objs, *dev_objs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    p = subprocess.run([exe, "40"], capture_output=True, text=True, env=env, timeout=600)
    assert p.returncode == 0, p.stdout + p.stderr[-4000:]
    assert "AddressSanitizer" not in p.stderr and "runtime error" not in p.stderr, p.stderr[-4000:]
    assert "; 0 failed checks" in p.stdout, p.stdout
    # the rounds did reach the code: plans built, tokens scheduled, adapters fetched
    m = re.search(r"(\d+) plans \((\d+) groups\), (\d+) scheduled tokens, (\d+) adapter", p.stdout)
    assert m and all(int(v) > 0 for v in m.groups()), p.stdout
