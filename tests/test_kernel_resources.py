"""Static resource check of every kernel instance in the built library (CPU only).

Reads the gfx950 code objects of our own build (the .hip_fatbin section of each
object under mamba_ssm_scan_amd/_build, unbundled with the ROCm LLVM tools) and,
from their metadata notes, each kernel's static LDS (group segment) and scratch
(private segment). Checks:
  * static LDS + the largest dynamic LDS a launch can request <= 160 KiB, the
    LDS of one gfx950 compute unit, for every instance;
  * no scratch (register spills) in the instances the workloads run on.
"""
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "mamba_ssm_scan_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
LDS_PER_CU = 160 * 1024

# the largest dynamic LDS each kernel that takes it can be launched with:
#   the generic fp32 prefill: 3 floats per token of a chunk (chunk <= 4096), or with the
#   chunk's turned B and C (and its masked scores) cached, at most 128 KiB in all;
#   the fused decode step's generic kernel: B_t and C_t rows, R * N <= 8192 floats each
DYNAMIC = {"prefill_generic_kernel": max(3 * 4096 * 4, 128 * 1024), "decode_generic_kernel": 2 * 8192 * 4}

# instances on the workloads' paths: no spills allowed
NO_SCRATCH = [r"prefill_ws_r1_kernelILb[01]ELb0ELi0ELb0E", r"prefill_ws4_kernelILi[248]ELb[01]ELb[01]ELb0E",
              r"decode_rows_kernel", r"decode_mfma(32)?_kernel", r"prologue_kernel"]


def _code_objects():
    objs = sorted(glob.glob(os.path.join(BUILD, "*.o")))
    if not objs or not os.path.exists(os.path.join(LLVM, "clang-offload-bundler")):
        pytest.skip("the library is not built here (run the build first) or the ROCm LLVM tools are missing")
    return objs


def _kernels(obj, tmp):
    fb = os.path.join(tmp, os.path.basename(obj) + ".fatbin")
    co = os.path.join(tmp, os.path.basename(obj) + ".co")
    r = subprocess.run([f"{LLVM}/llvm-objcopy", "--dump-section", f".hip_fatbin={fb}", obj, os.devnull],
                       capture_output=True, text=True)
    if r.returncode != 0:
        return []  # a host-only object
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    f"--input={fb}", f"--output={co}", "--unbundle"], check=True, capture_output=True)
    notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", co], check=True, capture_output=True,
                           text=True).stdout
    out, cur = [], {}
    for line in notes.splitlines():
        m = re.match(r"\s*\.(group_segment_fixed_size|private_segment_fixed_size|name):\s*(\S+)", line)
        if not m:
            continue
        cur[m.group(1)] = m.group(2)
        if len(cur) == 3:
            out.append((cur["name"], int(cur["group_segment_fixed_size"]), int(cur["private_segment_fixed_size"])))
            cur = {}
    return out


def test_lds_and_scratch_of_every_kernel(tmp_path):
    rows = []
    for obj in _code_objects():
        rows += [(os.path.basename(obj), *k) for k in _kernels(obj, str(tmp_path))]
    assert len(rows) > 50, "expected the library's kernel instances"
    over, spills = [], []
    for obj, name, lds, scratch in rows:
        dyn = max([v for k, v in DYNAMIC.items() if k in name] or [0])
        if lds + dyn > LDS_PER_CU:
            over.append(f"{name}: {lds} + {dyn} dynamic bytes")
        if scratch and any(re.search(p, name) for p in NO_SCRATCH):
            spills.append(f"{name}: {scratch} bytes of scratch")
    print(f"{len(rows)} kernel instances; largest static LDS {max(r[2] for r in rows)} bytes")
    assert not over, "LDS above 160 KiB:\n" + "\n".join(over)
    assert not spills, "spills in workload kernels:\n" + "\n".join(spills)
