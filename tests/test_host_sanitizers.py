"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the C entry points (m3_host.cpp, m3_mixer.cpp, m3_paths.cpp, with the
device launchers stubbed out: tests/host_check) and the fp64 oracle with gcc's
-fsanitize=address,undefined, then runs the ABI tests and the oracle's pins
against those builds in a child process that preloads libasan. Any sanitizer
report, and any stub reached (a device launch in a check that must not make
one), aborts the child and fails this test.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

def _load_builder():
    import importlib.util
    spec = importlib.util.spec_from_file_location("m3_host_check_build", os.path.join(HERE, "host_check", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


host_check = _load_builder()

SUITES = ["tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_prologue_pins.py",
          "tests/test_backward_pins.py", "tests/test_mixer_pins.py"]


def _have_toolchain():
    return all(os.path.exists(p) for p in ("/opt/rocm/lib/libamdhip64.so", "/opt/rocm/include/hip/hip_runtime.h"))


@pytest.mark.skipif(not _have_toolchain(), reason="HIP host headers and runtime library not installed")
def test_abi_and_oracle_pins_under_asan_ubsan(tmp_path):
    lib = host_check.build_host(str(tmp_path))
    orc = host_check.build_oracle(str(tmp_path))
    for so in (lib, orc):  # the builds really carry the instrumentation
        syms = subprocess.run(["nm", "-D", so], check=True, capture_output=True, text=True).stdout
        assert "__asan_report" in syms and "__ubsan_handle" in syms, so
    env = dict(os.environ)
    env.update(LD_PRELOAD=host_check.preload(), M3_LIBRARY=lib, M3_ORACLE_LIBRARY=orc,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *SUITES], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
