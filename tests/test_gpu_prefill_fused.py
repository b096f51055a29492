"""GPU parity of m3_prefill_fused: the prefill on the raw projections of the
step and the trapezoid weight (softplus with a per-head bias, sigmoid), mapped
where each kernel loads them.

Reference: oracle.prologue on the same raw dt / lambda bytes, then oracle.scan
with the problem's other inputs. Bar: the recurrence's own, max-relative per
(batch, head) slice (2e-2 bf16 I/O, 1e-4 fp32). The fused call is also held
against the unfused path (m3_prologue on dt and lambda, then m3_prefill) to the
same bar, on every path the plan can take: the 12-wave R 1 kernel, the
wave-specialised kernel at R 2, 4, 8 (and with sequence segments), the
general-pass MFMA kernel (other N, P), the token walk, and the fp32 generic
kernel.
"""
import os

import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close, f64, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # b, L, H, G, P, N, R, io, chunk, with lambda, with bias, what
    (2, 200, 3, 1, 64, 128, 1, "bf16", 64, True, True, "R 1, 12-wave kernel"),
    (1, 150, 2, 1, 64, 128, 2, "bf16", 64, True, True, "R 2, wave-specialised"),
    (2, 130, 2, 2, 64, 128, 4, "bf16", 64, True, True, "R 4, wave-specialised, two groups"),
    (1, 90, 2, 1, 64, 128, 8, "bf16", 64, True, True, "R 8, wave-specialised (32-token chunks)"),
    (1, 120, 2, 1, 32, 64, 1, "bf16", 64, True, True, "R 1, N 64 P 32: general-pass MFMA kernel"),
    (1, 70, 2, 1, 32, 64, 6, "bf16", 64, True, True, "R 6, N 64: token walk"),
    (1, 60, 2, 1, 8, 16, 1, "f32", 16, True, True, "fp32 generic"),
    (2, 140, 3, 1, 64, 128, 4, "bf16", 64, False, True, "R 4 without lambda (Euler)"),
    (2, 140, 3, 1, 64, 128, 1, "bf16", 64, True, False, "R 1 without dt bias"),
]


def _problem(b, L, H, G, P, N, R, io, wid):
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist="lm", wid=wid, h0_std=0.1, with_carry=True)
    raw = inputs.prologue_inputs(tokens=(b, L), heads=H, groups=G, rank=R, dstate=N, io_dtype=io, wid=wid + 1)
    return p, raw


def _run(p, raw, chunk, with_lam, with_bias, fused):
    d = to_dev(p)
    dt_raw = raw["dt_raw"].cuda()
    lam_raw = raw["lambda_raw"].cuda() if with_lam else None
    bias = raw["dt_bias"].cuda() if with_bias else None
    if fused:
        y, h = binding.prefill(d["x"], dt_raw, d["A"], d["omega"], lam_raw, d["B"], d["C"], d["D"], d["R"], chunk,
                               d.get("h0"), carry_B=d.get("carry_B"), carry_x=d.get("carry_x"), raw_steps=True,
                               dt_bias=bias)
    else:
        _, _, dt, lam = binding.prologue(dt_raw=dt_raw, dt_bias=bias, lambda_raw=lam_raw)
        y, h = binding.prefill(d["x"], dt, d["A"], d["omega"], lam, d["B"], d["C"], d["D"], d["R"], chunk,
                               d.get("h0"), carry_B=d.get("carry_B"), carry_x=d.get("carry_x"))
    torch.cuda.synchronize()
    return y, h


def _oracle(p, raw, with_lam, with_bias):
    ref = oracle.prologue(dt_raw=f64(raw["dt_raw"]), dt_bias=f64(raw["dt_bias"]) if with_bias else None,
                          lambda_raw=f64(raw["lambda_raw"]) if with_lam else None)
    q = dict(p)
    q["dt"] = torch.from_numpy(ref["dt"])
    # no lambda: the Euler rule, lambda = 1 for every token
    q["lam"] = torch.from_numpy(ref["lambda"]) if with_lam else torch.ones_like(q["dt"])
    return oracle.scan(q)


@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_prefill_fused_steps(case):
    b, L, H, G, P, N, R, io, chunk, with_lam, with_bias, _ = case
    print(f"fused prefill case {case}", flush=True)
    p, raw = _problem(b, L, H, G, P, N, R, io, 5000 + CASES.index(case))
    y_ref, h_ref = _oracle(p, raw, with_lam, with_bias)
    y, h = _run(p, raw, chunk, with_lam, with_bias, fused=True)
    tol = TOL[io]
    assert_close(y, y_ref, tol, "y (fused) vs oracle")
    assert_close(h, h_ref, tol, "h_out (fused) vs oracle")
    yu, hu = _run(p, raw, chunk, with_lam, with_bias, fused=False)
    assert_close(y, f64(yu), tol, "y fused vs prologue + prefill")
    assert_close(h, f64(hu), tol, "h_out fused vs prologue + prefill")


def test_prefill_fused_with_segments():
    """The long-sequence layout (few walks, sequence segments joined by look-back) on raw steps."""
    b, L, H, G, P, N, R = 1, 1100, 2, 1, 64, 128, 4
    p, raw = _problem(b, L, H, G, P, N, R, "bf16", 5100)
    old = os.environ.get("M3_PREFILL_SEGMENTS")
    os.environ["M3_PREFILL_SEGMENTS"] = "3"
    try:
        plan = binding.plan(binding.dims(b, L, H, G, P, N), R, 64, binding.M3_BF16)
        assert plan.segments == 3
        y, h = _run(p, raw, 64, True, True, fused=True)
    finally:
        if old is None:
            del os.environ["M3_PREFILL_SEGMENTS"]
        else:
            os.environ["M3_PREFILL_SEGMENTS"] = old
    y_ref, h_ref = _oracle(p, raw, True, True)
    assert_close(y, y_ref, TOL["bf16"], "y (fused, 3 segments) vs oracle")
    assert_close(h, h_ref, TOL["bf16"], "h_out (fused, 3 segments) vs oracle")
