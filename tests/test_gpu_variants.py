"""GPU parity of the special cases omega = 0 and lambda = 1, passed as NULL arrays.

omega NULL: real-valued state, no rotation (the R = 1 prefill runs a kernel
instance without RoPE); lambda NULL: the Euler rule (no previous-input term),
which the pages identify with Mamba-2. Every path is covered: bf16 MFMA prefill
at R 1, 2, 4, the fp32 generic prefill, and the decode kernels (R 1 float4,
R 2/4 MFMA, generic). The oracle runs the same problem with omega = 0 and
lambda = 1 written out as arrays.
"""
import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close, to_dev

pytestmark = pytest.mark.gpu


def _ref(p, no_omega, no_lam):
    q = dict(p)
    if no_omega:
        q["omega"] = torch.zeros_like(p["omega"])
    if no_lam:
        q["lam"] = torch.ones_like(p["lam"])
    return oracle.scan(q)


PCASES = [
    # b, L, H, G, P, N, R, io, chunk, omega NULL, lambda NULL
    (2, 200, 3, 1, 64, 128, 1, "bf16", 64, True, False),
    (1, 257, 2, 1, 64, 128, 1, "bf16", 64, False, True),
    (2, 150, 2, 1, 64, 128, 1, "bf16", 64, True, True),
    (1, 190, 2, 1, 64, 128, 4, "bf16", 64, True, True),
    (1, 100, 2, 2, 64, 128, 2, "bf16", 32, True, False),
    (1, 90, 2, 1, 8, 16, 1, "f32", 16, True, True),
    (2, 70, 3, 3, 8, 16, 2, "f32", 16, False, True),
]


@pytest.mark.parametrize("case", PCASES, ids=[str(c) for c in PCASES])
def test_prefill_special_cases(case):
    b, L, H, G, P, N, R, io, chunk, no_om, no_lam = case
    print(f"prefill special case {case}", flush=True)
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist="lm", wid=900 + PCASES.index(case), h0_std=0.1, with_carry=True)
    y_ref, h_ref = _ref(p, no_om, no_lam)
    d = to_dev(p)
    y, h = binding.prefill(d["x"], d["dt"], d["A"], None if no_om else d["omega"], None if no_lam else d["lam"],
                           d["B"], d["C"], d["D"], R, chunk, d["h0"], carry_B=d["carry_B"], carry_x=d["carry_x"])
    torch.cuda.synchronize()
    assert_close(y, y_ref, TOL[io], "y")
    assert_close(h, h_ref, TOL[io], "h_out")


DCASES = [
    # b, L, H, G, P, N, R, io, omega NULL, lambda NULL
    (2, 10, 4, 1, 64, 128, 1, "bf16", True, True),
    (2, 10, 4, 1, 64, 128, 4, "bf16", True, False),
    (1, 8, 3, 3, 64, 128, 2, "bf16", False, True),
    (2, 9, 2, 1, 8, 16, 2, "f32", True, True),
]


@pytest.mark.parametrize("case", DCASES, ids=[str(c) for c in DCASES])
def test_decode_special_cases(case):
    b, L, H, G, P, N, R, io, no_om, no_lam = case
    print(f"decode special case {case}", flush=True)
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist="lm", wid=950 + DCASES.index(case), h0_std=0.1, with_carry=True)
    y_ref, h_ref = _ref(p, no_om, no_lam)
    d = to_dev(p)
    st = binding.DecodeState(b, H, G, P, N, R, io_dtype=d["x"].dtype, h0=d["h0"], B_last=d["carry_B"],
                             x_last=d["carry_x"])
    ys = []
    for t in range(L):
        ys.append(st.step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                          None if no_om else d["omega"], None if no_lam else d["lam"][:, t].contiguous(),
                          d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d["D"]))
    torch.cuda.synchronize()
    assert_close(torch.stack(ys, 1), y_ref, TOL[io], "decode y")
    assert_close(st.h, h_ref, TOL[io], "decode h")
