"""GPU parity at the larger deployment sizes: state dimension N = 256 and MIMO
ranks R = 6 and 8 (the state-size and rank knobs of "Mamba-3架构技术解析" §4.3
and the MIMO rank of "复值SSM × 广义梯形离散 × MIMO" §2.3).

These shapes run on the generic kernels (chunked fp32 prefill, generic decode
step): the MFMA prefill is built for N 128, P 64, R 1/2/4. The oracle runs the
same problem in fp64; bars are the recurrence's own (1e-4 fp32, 2e-2 bf16 I/O,
max-relative per (batch, head) slice).
"""
import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close, gpu_prefill, to_dev

pytestmark = pytest.mark.gpu

PCASES = [
    # b, L, H, G, P, N, R, io, chunk
    (1, 150, 2, 1, 64, 256, 1, "bf16", 64),   # N 256, ragged last chunk
    (2, 70, 2, 1, 64, 128, 8, "bf16", 32),    # R 8
    (1, 90, 3, 3, 64, 256, 6, "bf16", 64),    # N 256 and R 6, one B, C per head
    (1, 45, 2, 1, 16, 256, 8, "f32", 16),     # fp32, both large
]


@pytest.mark.parametrize("case", PCASES, ids=[str(c) for c in PCASES])
def test_prefill_large_state_and_rank(case):
    b, L, H, G, P, N, R, io, chunk = case
    print(f"prefill large case {case}", flush=True)
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist="lm", wid=1000 + PCASES.index(case), h0_std=0.1, with_carry=True)
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert_close(y, y_ref, TOL[io], "y")
    assert_close(h, h_ref, TOL[io], "h_out")


DCASES = [
    # b, L, H, G, P, N, R, io
    (2, 8, 2, 1, 64, 256, 1, "bf16"),
    (2, 8, 2, 1, 64, 128, 8, "bf16"),
    (1, 6, 3, 3, 64, 256, 6, "f32"),
]


@pytest.mark.parametrize("case", DCASES, ids=[str(c) for c in DCASES])
def test_decode_large_state_and_rank(case):
    b, L, H, G, P, N, R, io = case
    print(f"decode large case {case}", flush=True)
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist="lm", wid=1050 + DCASES.index(case), h0_std=0.1, with_carry=True)
    y_ref, h_ref = oracle.scan(p)
    d = to_dev(p)
    st = binding.DecodeState(b, H, G, P, N, R, io_dtype=d["x"].dtype, h0=d["h0"], B_last=d["carry_B"],
                             x_last=d["carry_x"])
    ys = [st.step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"], d["omega"],
                  d["lam"][:, t].contiguous(), d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d["D"])
          for t in range(L)]
    torch.cuda.synchronize()
    assert_close(torch.stack(ys, 1), y_ref, TOL[io], "decode y")
    assert_close(st.h, h_ref, TOL[io], "decode h")


def test_prefill_then_decode_large():
    """N 256, R 8: a prefill of 40 tokens handed to the decode state, 6 more steps, against one 46-token walk."""
    b, L, H, G, P, N, R, io, k = 1, 46, 2, 1, 32, 256, 8, "bf16", 40
    print("prefill + decode handoff, N 256, R 8", flush=True)
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist="lm", wid=1080, h0_std=0.1)
    y_ref, h_ref = oracle.scan(p)
    d = to_dev(p)
    pre = {kk: (v[:, :k].contiguous() if kk in ("x", "B", "C", "dt", "lam") else v) for kk, v in d.items()}
    y0, h0 = gpu_prefill(pre, 32)
    st = binding.DecodeState(b, H, G, P, N, R, io_dtype=d["x"].dtype, h0=h0, B_last=d["B"][:, k - 1].contiguous(),
                             x_last=d["x"][:, k - 1].contiguous(), t0=k)
    ys = [st.step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"], d["omega"],
                  d["lam"][:, t].contiguous(), d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d["D"])
          for t in range(k, L)]
    torch.cuda.synchronize()
    assert_close(torch.cat([y0.cpu(), torch.stack(ys, 1).cpu()], 1), y_ref, TOL[io], "y")
    assert_close(st.h, h_ref, TOL[io], "h")
