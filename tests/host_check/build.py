"""Host-only builds with AddressSanitizer and UndefinedBehaviorSanitizer (gcc):

* libm3_hostcheck.so -- the C entry points (m3_host.cpp, m3_mixer.cpp,
  m3_paths.cpp) with the device launchers replaced by the stubs of
  m3_stub_launch.cpp, linked against the HIP runtime and hipBLASLt host
  libraries (no GPU is touched: the tests that load it stop at argument checks);
* libm3oracle_check.so -- the fp64 oracle.

Both use gcc's sanitizer runtimes; a process that loads them must preload
libasan (`preload()`).
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "mamba_ssm_scan_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]


def build_host(outdir: str) -> str:
    out = os.path.join(outdir, "libm3_hostcheck.so")
    srcs = [os.path.join(CSRC, f) for f in ("m3_host.cpp", "m3_mixer.cpp", "m3_paths.cpp")]
    srcs.append(os.path.join(HERE, "m3_stub_launch.cpp"))
    cmd = ["g++", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", out, *srcs,
           "-L/opt/rocm/lib", "-lamdhip64", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def build_oracle(outdir: str) -> str:
    out = os.path.join(outdir, "libm3oracle_check.so")
    cmd = ["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", *SAN, "-o", out,
           os.path.join(ROOT, "oracle", "m3_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def preload() -> str:
    """Path of gcc's libasan, to put in LD_PRELOAD."""
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True, capture_output=True,
                          text=True).stdout.strip()
