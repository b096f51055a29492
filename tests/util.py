"""Shared helpers for the GPU parity tests (device moves, tolerances, comparisons)."""
import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}   # max-relative error per (batch, head) slice

# every comparison made in this process: (test id, what, error, tolerance); the
# session summary prints the full-size ones and the worst error / tolerance ratio
ERRORS = []


def to_dev(p, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def to_host(p):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def gpu_prefill(p, chunk, **kw):
    from mamba_ssm_scan_amd import binding
    d = to_dev(p)
    y, h = binding.prefill(d["x"], d["dt"], d["A"], d["omega"], d["lam"], d["B"], d["C"], d["D"], d["R"], chunk,
                           d.get("h0"), carry_B=d.get("carry_B"), carry_x=d.get("carry_x"), **kw)
    torch.cuda.synchronize()
    return y, h


def assert_close(got, ref, tol, what=""):
    import os
    err = oracle.max_rel_err(f64(got) if isinstance(got, torch.Tensor) else got, ref)
    print(f"  {what}: max-rel error {err:.3e} (tol {tol:.0e})", flush=True)
    ERRORS.append((os.environ.get("PYTEST_CURRENT_TEST", "?").split(" (")[0], what, float(err), float(tol)))
    assert np.isfinite(err) and err <= tol, f"{what}: max-rel error {err:.3e} > {tol:.1e}"
    return err
