"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the CPU-side code
(no GPU):

* the oracle (``oracle/moe_oracle.c``) under gcc's ASan + UBSan, driven by
  ``oracle/sanitize_check.c`` over every format, routing mode and feature
  flag on small ragged layers whose arrays are allocated at their exact
  sizes, with leak detection;
* the library's host translation unit (plan, layout, argument checks) built
  with the sanitizers on its host side only, linked with the ordinary kernel
  objects, and driven by ``tests/host_abi_check.cpp`` through thousands of
  plans and every rejection path of the forwards (each returns before a
  launch).

Any sanitizer report aborts its run (``-fno-sanitize-recover=all``).
"""
import glob
import os
import subprocess

import pytest

from mixture_experts_decode_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
OUT = os.path.join(ROOT, "_build", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
# For hipcc the sanitizers go to the host compilation only.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}...: rc {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r.stdout


def test_oracle_under_address_and_undefined_behaviour_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_check")
    _run(["gcc", "-std=c11", "-g", "-O1", *SAN, "-fopenmp", "-I", ORACLE,
          os.path.join(ORACLE, "sanitize_check.c"), os.path.join(ORACLE, "moe_oracle.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    assert _run([exe], env=env).startswith("ok")


def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    objs = {os.path.basename(p) for p in glob.glob(os.path.join(hip_build.OBJDIR, "*.o"))}
    srcs = {os.path.basename(p) + ".o" for p in glob.glob(os.path.join(hip_build.CSRC, "*.hip"))}
    if not srcs <= objs:
        hip_build.build()
    flags = [f for f in hip_build.CFLAGS if f != "-O3"] + ["-O1", "-g"]
    host_obj = os.path.join(OUT, "moe_decode_host_san.o")
    _run([hip_build.HIPCC, *flags, *HOST_SAN, "-c", os.path.join(hip_build.CSRC, "moe_decode_host.hip"),
          "-o", host_obj])
    drv_obj = os.path.join(OUT, "host_abi_check.o")
    _run([hip_build.HIPCC, "-O1", "-g", "-std=c++17", *HOST_SAN, "-I", hip_build.INCLUDE, "-c",
          os.path.join(ROOT, "tests", "host_abi_check.cpp"), "-o", drv_obj])
    kernels = sorted(p for p in glob.glob(os.path.join(hip_build.OBJDIR, "*.o"))
                     if os.path.basename(p) != "moe_decode_host.hip.o")
    exe = os.path.join(OUT, "host_abi_check")
    _run([hip_build.HIPCC, f"--offload-arch={hip_build.ARCH}", *HOST_SAN, drv_obj, host_obj, *kernels, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("HIP_VISIBLE_DEVICES", None)
    assert _run([exe], env=env).startswith("ok")
