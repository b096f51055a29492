"""CPU fp64 oracle for the Mamba-3 SSM recurrence -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. It wraps `m3_oracle.c` (plain C, double precision, OpenMP over
(batch, head)) through ctypes; see that file for the recurrence it runs and
the passages of the pages it follows. The input prologue (QK-norm and bias on
B and C, softplus / sigmoid on the step and the trapezoid weight) is the numpy
module `prologue.py`. Nothing here is shared with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .prologue import prologue, qk_norm, rms_rows, sigmoid, softplus  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m3_oracle.c")
_LIB = os.path.join(_HERE, "libm3oracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (-O3, no fast-math, OpenMP)."""
    cmd = ["gcc", "-O3", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("M3_ORACLE_LIBRARY")  # another build of the oracle (the sanitizer check)
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        lib = ctypes.CDLL(path)
        f = lib.m3o_scan
        i64 = ctypes.c_int64
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        f.argtypes = [i64] * 7 + [fp] * 11 + [dp, dp, ctypes.c_int]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, n)


def _f32(a):
    """Exact single-precision carrier of a torch tensor or array (bf16 widens exactly)."""
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a, ctype):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(ctype))
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def scan(p: dict, nthreads: int | None = None):
    """Run the sequential recurrence over a problem dict (see mamba_ssm_scan_amd.inputs).

    Returns (y, h_out) as float64 numpy arrays, y [b][L][H][R][P], h_out [b][H][N][P].
    """
    lib = _load()
    x = _f32(p["x"])
    dt = _f32(p["dt"])
    lam = _f32(p["lam"])
    B = _f32(p["B"])
    C = _f32(p["C"])
    A = _f32(p["A"])
    om = _f32(p["omega"])
    D = _f32(p["D"])
    h0 = _f32(p.get("h0"))
    cB = _f32(p.get("carry_B"))
    cx = _f32(p.get("carry_x"))
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    if B.shape != (b, L, G, R, N) or C.shape != B.shape:
        raise ValueError("B/C shape mismatch")
    if dt.shape != (b, L, H) or lam.shape != (b, L, H):
        raise ValueError("dt/lambda shape mismatch")
    if A.shape != (H,) or D.shape != (H,) or om.shape != (H, N // 2):
        raise ValueError("per-head parameter shape mismatch")
    if h0 is not None and h0.shape != (b, H, N, P):
        raise ValueError("h0 shape mismatch")
    if cB is not None and cB.shape != (b, G, R, N):
        raise ValueError("carry_B shape mismatch")
    if cx is not None and cx.shape != (b, H, R, P):
        raise ValueError("carry_x shape mismatch")
    y = np.empty((b, L, H, R, P), dtype=np.float64)
    h_out = np.empty((b, H, N, P), dtype=np.float64)
    rc = lib.m3o_scan(b, L, H, G, P, N, R,
                      _ptr(x, ctypes.c_float), _ptr(dt, ctypes.c_float), _ptr(A, ctypes.c_float),
                      _ptr(om, ctypes.c_float), _ptr(lam, ctypes.c_float), _ptr(B, ctypes.c_float),
                      _ptr(C, ctypes.c_float), _ptr(D, ctypes.c_float), _ptr(h0, ctypes.c_float),
                      _ptr(cB, ctypes.c_float), _ptr(cx, ctypes.c_float),
                      _ptr(y, ctypes.c_double), _ptr(h_out, ctypes.c_double),
                      nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return y, h_out


def max_rel_err(got, ref) -> float:
    """max over (batch, head) slices of max|got - ref| / max|ref|.

    Arrays are [b][L][H][...] (y) or [b][H][...] (state); the slice axes are
    (0, 2) for rank-5 y arrays and (0, 1) for rank-4 states.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {ref.shape}")
    if ref.ndim == 5:  # y: [b][L][H][R][P] -> [b][H][L*R*P]
        g = np.moveaxis(got, 2, 1).reshape(ref.shape[0], ref.shape[2], -1)
        r = np.moveaxis(ref, 2, 1).reshape(ref.shape[0], ref.shape[2], -1)
    else:
        g = got.reshape(ref.shape[0], ref.shape[1], -1)
        r = ref.reshape(ref.shape[0], ref.shape[1], -1)
    if g.size == 0:
        return 0.0
    num = np.abs(g - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(rel.max())
