"""GPU parity of m3_prologue (the input prologue) against the fp64 oracle.

The HIP kernel computes in fp32 and rounds B, C to the I/O dtype; the oracle
(oracle/prologue.py) runs the same formulas in fp64. Bars:
  B, C  per (token, group, rank) row: max |gpu - ref| / max |ref| <= 2^-7
        for bf16 output (one rounding to bf16 is at most 2^-8 relative to the
        value, reached just above a power of two; the fp32 arithmetic before
        it adds ~1e-7, so the bar leaves a factor 2), <= 1e-5 for fp32;
  dt, lambda  max |gpu - ref| / |ref| <= 1e-5 (fp32 exp / log1p).
End to end, prologue -> m3_prefill is held to the recurrence's bars against
oracle.prologue -> oracle.scan on the same raw bytes.
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_ssm_scan_amd import inputs
from tests.util import TOL, assert_close, f64

pytestmark = pytest.mark.gpu


def _ref(p, parts=("B", "C", "dt", "lambda"), weights=True):
    n = lambda k: None if p.get(k) is None else f64(p[k])
    return oracle.prologue(B_raw=n("B_raw") if "B" in parts else None, C_raw=n("C_raw") if "C" in parts else None,
                           B_weight=n("B_weight") if weights else None, B_bias=n("B_bias") if weights else None,
                           C_weight=n("C_weight") if weights else None, C_bias=n("C_bias") if weights else None,
                           eps=p["eps"], dt_raw=n("dt_raw") if "dt" in parts else None,
                           dt_bias=n("dt_bias") if weights else None,
                           lambda_raw=n("lambda_raw") if "lambda" in parts else None)


def _check_rows(got, ref, io, what):
    g, r = f64(got), ref
    g = g.reshape(-1, g.shape[-1])
    r = r.reshape(-1, r.shape[-1])
    den = np.abs(r).max(axis=1)
    err = float((np.abs(g - r).max(axis=1) / np.where(den > 0, den, 1.0)).max()) if r.size else 0.0
    tol = 2.0 ** -7 if io == "bf16" else 1e-5
    print(f"  {what}: row max-rel {err:.3e} (tol {tol:.1e})", flush=True)
    assert err <= tol, f"{what}: {err:.3e} > {tol:.1e}"


def _check_scalars(got, ref, what):
    g, r = f64(got), ref
    err = float((np.abs(g - r) / np.abs(r)).max()) if r.size else 0.0
    print(f"  {what}: max rel {err:.3e}", flush=True)
    assert err <= 1e-5, f"{what}: {err:.3e}"


def _dev(p):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def _gpu(p, weights=True, **kw):
    from mamba_ssm_scan_amd import binding
    d = _dev(p)
    w = (lambda k: d[k]) if weights else (lambda k: None)
    out = binding.prologue(d["B_raw"], d["C_raw"], B_weight=w("B_weight"), B_bias=w("B_bias"),
                           C_weight=w("C_weight"), C_bias=w("C_bias"), eps=p["eps"], dt_raw=d["dt_raw"],
                           dt_bias=w("dt_bias"), lambda_raw=d["lambda_raw"], **kw)
    torch.cuda.synchronize()
    return out


CASES = [
    # tokens, H, G, R, N, io
    ((3, 37), 8, 2, 3, 128, "bf16"),   # 16-lane rows of 8-entry pieces, ragged row count
    ((3, 37), 8, 2, 3, 128, "f32"),
    ((2, 9), 6, 3, 2, 264, "bf16"),    # N above 128: a second and a partial third piece
    ((5,), 4, 1, 1, 6, "f32"),         # N not a multiple of 8: one entry per lane and step
    ((5,), 4, 1, 1, 6, "bf16"),
    ((4, 2048), 64, 1, 4, 128, "bf16"),  # the R 4 prefill workload's shapes, compared in full
]


@pytest.mark.parametrize("tokens,H,G,R,N,io", CASES)
def test_prologue_matches_oracle(tokens, H, G, R, N, io):
    print(f"case tokens={tokens} H={H} G={G} R={R} N={N} io={io}", flush=True)
    p = inputs.prologue_inputs(tokens=tokens, heads=H, groups=G, rank=R, dstate=N, io_dtype=io, wid=201)
    p["eps"] = 1e-6
    ref = _ref(p)
    B, C, dt, lam = _gpu(p)
    _check_rows(B, ref["B"], io, "B")
    _check_rows(C, ref["C"], io, "C")
    _check_scalars(dt, ref["dt"], "dt")
    _check_scalars(lam, ref["lambda"], "lambda")


def test_prologue_without_weights_and_in_place():
    from mamba_ssm_scan_amd import binding
    p = inputs.prologue_inputs(tokens=(2, 33), heads=4, groups=1, rank=2, dstate=128, io_dtype="bf16", wid=202)
    p["eps"] = 0.0
    ref = _ref(p, weights=False)
    d = _dev(p)
    B, C, dt, lam = d["B_raw"].clone(), d["C_raw"].clone(), d["dt_raw"].clone(), d["lambda_raw"].clone()
    binding.prologue(B, C, eps=0.0, dt_raw=dt, lambda_raw=lam, B=B, C=C, dt=dt, lam=lam)
    torch.cuda.synchronize()
    _check_rows(B, ref["B"], "bf16", "B in place")
    _check_rows(C, ref["C"], "bf16", "C in place")
    _check_scalars(dt, ref["dt"], "dt in place")
    _check_scalars(lam, ref["lambda"], "lambda in place")
    # weight 1, bias 0, eps 0: every row has unit mean square up to bf16 rounding
    ms = (f64(B) ** 2).mean(axis=-1)
    assert np.abs(ms - 1).max() < 2 ** -7


def test_prologue_parts_and_edges():
    from mamba_ssm_scan_amd import binding
    p = inputs.prologue_inputs(tokens=(7,), heads=2, groups=1, rank=1, dstate=16, io_dtype="f32", wid=203)
    d = _dev(p)
    # dt only (lambda untouched elsewhere)
    _, _, dt, lam = binding.prologue(dt_raw=d["dt_raw"], dt_bias=d["dt_bias"])
    torch.cuda.synchronize()
    assert lam is None
    _check_scalars(dt, oracle.prologue(dt_raw=f64(p["dt_raw"]), dt_bias=f64(p["dt_bias"]))["dt"], "dt only")
    # zero rows stay finite with eps > 0 and become the bias
    z = torch.zeros_like(d["B_raw"])
    B, _, _, _ = binding.prologue(z, B_bias=d["B_bias"], eps=1e-6)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(B), np.broadcast_to(f64(p["B_bias"]), B.shape))
    # extreme raw steps: softplus stays finite and positive, sigmoid in [0, 1]
    ext = torch.tensor([[-100.0, 100.0], [-20.0, 20.0], [0.0, 1e-30]], device="cuda")
    _, _, dt, lam = binding.prologue(dt_raw=ext, lambda_raw=ext)
    torch.cuda.synchronize()
    ref = oracle.prologue(dt_raw=f64(ext), lambda_raw=f64(ext))
    np.testing.assert_allclose(f64(dt), ref["dt"], rtol=1e-5, atol=1e-38)  # softplus(-100) is an fp32 denormal
    np.testing.assert_allclose(f64(lam), ref["lambda"], rtol=1e-5, atol=1e-38)
    # no tokens: nothing launched, nothing to check but the call
    empty = torch.empty((0, 1, 1, 16), device="cuda")
    binding.prologue(empty)


@pytest.mark.parametrize("R", [1, 4])
def test_prologue_then_prefill_matches_oracle(R):
    """Raw projections -> m3_prologue -> m3_prefill against oracle.prologue -> oracle.scan.

    The oracle side rounds its B, C to bf16 (the I/O dtype both sides hand to
    the recurrence) and its dt, lambda to fp32.
    """
    from mamba_ssm_scan_amd import binding
    b, L, H, G, P, N = 2, 200, 4, 1, 64, 128
    print(f"case prologue+prefill R={R}", flush=True)
    raw = inputs.prologue_inputs(tokens=(b, L), heads=H, groups=G, rank=R, dstate=N, io_dtype="bf16", wid=204)
    raw["eps"] = 1e-6
    rest = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R,
                               io_dtype="bf16", dist="lm", wid=205)
    ref = _ref(raw)
    p_ref = dict(rest)
    p_ref["B"] = torch.from_numpy(ref["B"]).to(torch.bfloat16)
    p_ref["C"] = torch.from_numpy(ref["C"]).to(torch.bfloat16)
    p_ref["dt"] = torch.from_numpy(ref["dt"]).to(torch.float32)
    p_ref["lam"] = torch.from_numpy(ref["lambda"]).to(torch.float32)
    y_ref, h_ref = oracle.scan(p_ref)

    B, C, dt, lam = _gpu(raw)
    d = _dev(rest)
    y, h = binding.prefill(d["x"], dt, d["A"], d["omega"], lam, B, C, d["D"], R, 64)
    torch.cuda.synchronize()
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")
