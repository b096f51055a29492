"""GPU parity of m3_decode_step_fused: the decode step on the raw projections,
with the input prologue (QK-norm, weight and bias on B_t and C_t, softplus with
the head's bias on the step, sigmoid on lambda) computed in the step kernel.

Reference: oracle.prologue on the same raw bytes, then oracle.scan over the
steps (the decode loop is the recurrence over the step axis from h0 with zero
carries). Bar: the recurrence's own, max-relative per (batch, head) slice
(2e-2 bf16 I/O, 1e-4 fp32). The fused step is also held against the unfused
path (m3_prologue into buffers, then m3_decode_step) to the same bar.
"""
import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close, f64

pytestmark = pytest.mark.gpu

CASES = [
    # b, H, G, P, N, R, io, steps, which kernel
    (3, 4, 1, 64, 128, 1, "bf16", 6, "rows, R 1"),
    (2, 4, 2, 64, 128, 4, "bf16", 5, "MFMA, R 4, two groups"),
    (2, 2, 1, 64, 128, 2, "bf16", 4, "MFMA, R 2"),
    (1, 3, 1, 64, 64, 8, "bf16", 4, "MFMA, R 8, N 64"),
    (2, 2, 2, 32, 256, 3, "bf16", 4, "rows, N 256, P 32, R 3"),
    (1, 2, 1, 16, 32, 2, "f32", 5, "generic, fp32"),
    (2, 3, 3, 8, 16, 5, "bf16", 4, "generic, R 5"),
]


def _problem(b, H, G, P, N, R, io, steps, wid):
    dt_ = torch.bfloat16 if io == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(wid)
    per = [inputs.prologue_inputs(tokens=(b,), heads=H, groups=G, rank=R, dstate=N, io_dtype=io, wid=wid, step=t)
           for t in range(steps)]
    x = torch.randn((steps, b, H, R, P), generator=g).to(dt_)
    A = -torch.exp(torch.empty(H).uniform_(0.0, 2.0, generator=g))
    omega = torch.empty((H, N // 2)).uniform_(0.0, 3.14159, generator=g)
    D = 1.0 + 0.1 * torch.randn(H, generator=g)
    h0 = 0.1 * torch.randn((b, H, N, P), generator=g)
    return per, x, A, omega, D, h0


@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_decode_fused_prologue(case):
    b, H, G, P, N, R, io, steps, _ = case
    print(f"fused decode case {case}", flush=True)
    per, x, A, omega, D, h0 = _problem(b, H, G, P, N, R, io, steps, 4000 + CASES.index(case))
    dev = lambda t: t.cuda()
    eps = 1e-6
    st = binding.DecodeState(b, H, G, P, N, R, io_dtype=x.dtype, h0=dev(h0))
    ys = []
    for t in range(steps):
        p = per[t]
        ys.append(st.step_fused(dev(x[t]), dev(p["dt_raw"]), dev(A), dev(omega), dev(p["lambda_raw"]),
                                dev(p["B_raw"]), dev(p["C_raw"]), dev(D), dt_bias=dev(p["dt_bias"]),
                                B_weight=dev(p["B_weight"]), B_bias=dev(p["B_bias"]), C_weight=dev(p["C_weight"]),
                                C_bias=dev(p["C_bias"]), eps=eps))
    torch.cuda.synchronize()
    y = torch.stack(ys, 1)  # [b][steps][H][R][P]

    # the oracle: prologue on the same raw bytes, then the recurrence over the steps
    refs = [oracle.prologue(B_raw=f64(p["B_raw"]), C_raw=f64(p["C_raw"]), B_weight=f64(p["B_weight"]),
                            B_bias=f64(p["B_bias"]), C_weight=f64(p["C_weight"]), C_bias=f64(p["C_bias"]), eps=eps,
                            dt_raw=f64(p["dt_raw"]), dt_bias=f64(p["dt_bias"]), lambda_raw=f64(p["lambda_raw"]))
            for p in per]
    stack = lambda k: torch.tensor([r[k] for r in refs]).transpose(0, 1).contiguous()  # [b][steps]...
    prob = {"x": x.transpose(0, 1).contiguous(), "B": stack("B"), "C": stack("C"), "dt": stack("dt"),
            "lam": stack("lambda"), "A": A, "omega": omega, "D": D, "h0": h0, "R": R, "io_dtype": io,
            "carry_B": None, "carry_x": None}
    y_ref, h_ref = oracle.scan(prob)
    assert_close(y, y_ref, TOL[io], f"y over {steps} fused steps")
    assert_close(st.h, h_ref, TOL[io], "state after the fused steps")

    # the unfused path on the same raw inputs: m3_prologue, then m3_decode_step
    st2 = binding.DecodeState(b, H, G, P, N, R, io_dtype=x.dtype, h0=dev(h0))
    ys2 = []
    for t in range(steps):
        p = per[t]
        Bn, Cn, dtn, lamn = binding.prologue(dev(p["B_raw"]), dev(p["C_raw"]), B_weight=dev(p["B_weight"]),
                                             B_bias=dev(p["B_bias"]), C_weight=dev(p["C_weight"]),
                                             C_bias=dev(p["C_bias"]), eps=eps, dt_raw=dev(p["dt_raw"]),
                                             dt_bias=dev(p["dt_bias"]), lambda_raw=dev(p["lambda_raw"]))
        ys2.append(st2.step(dev(x[t]), dtn, dev(A), dev(omega), lamn, Bn, Cn, dev(D)))
    torch.cuda.synchronize()
    y2 = torch.stack(ys2, 1)
    assert_close(y, f64(y2), TOL[io], "fused against m3_prologue + m3_decode_step")


def test_decode_fused_without_lambda_and_weights():
    """lambda_raw NULL (lambda = 1) and no weights / biases (unit weight, zero bias, no dt bias)."""
    b, H, G, P, N, R, steps = 2, 2, 1, 64, 128, 4, 3
    print("fused decode without lambda / weights", flush=True)
    per, x, A, omega, D, h0 = _problem(b, H, G, P, N, R, "bf16", steps, 4100)
    dev = lambda t: t.cuda()
    st = binding.DecodeState(b, H, G, P, N, R, io_dtype=x.dtype, h0=dev(h0))
    ys = [st.step_fused(dev(x[t]), dev(per[t]["dt_raw"]), dev(A), dev(omega), None, dev(per[t]["B_raw"]),
                        dev(per[t]["C_raw"]), dev(D), eps=1e-6) for t in range(steps)]
    torch.cuda.synchronize()
    refs = [oracle.prologue(B_raw=f64(p["B_raw"]), C_raw=f64(p["C_raw"]), eps=1e-6, dt_raw=f64(p["dt_raw"]))
            for p in per]
    stack = lambda k: torch.tensor([r[k] for r in refs]).transpose(0, 1).contiguous()
    prob = {"x": x.transpose(0, 1).contiguous(), "B": stack("B"), "C": stack("C"), "dt": stack("dt"),
            "lam": torch.ones((b, steps, H)), "A": A, "omega": omega, "D": D, "h0": h0, "R": R,
            "io_dtype": "bf16", "carry_B": None, "carry_x": None}
    y_ref, h_ref = oracle.scan(prob)
    assert_close(torch.stack(ys, 1), y_ref, TOL["bf16"], "y, lambda = 1, unit weights")
    assert_close(st.h, h_ref, TOL["bf16"], "state")
