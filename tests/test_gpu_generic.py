"""GPU parity of the generic (any-shape, fp32-arithmetic) prefill and of the decode
step against the CPU oracle, plus exact bookkeeping checks.

Tolerances: max-relative error per (batch, head) slice <= 1e-4 with fp32 I/O and
<= 2e-2 with bf16 I/O; exact equality where the arithmetic is exact (dyadic case).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from mamba_ssm_scan_amd import inputs
from tests.util import TOL, assert_close, f64, gpu_prefill, to_dev

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def test_workload0_prefill_chunk16():
    p = inputs.workload_prefill(0)
    _flush("workload 0 prefill, chunk 16")
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, 16)
    assert_close(y, y_ref, 1e-4, "y")
    assert_close(h, h_ref, 1e-4, "h_out")


# the generic kernel's three forms (workload 0: R 1, N 16): up to chunk 128 the
# chunk's turned B, C and masked scores fit its LDS cache, at 200 the turned B
# and C only, at 4096 neither (the turns are recomputed where they are used)
@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 7, 16, 64, 127, 128, 200, 4096])
def test_workload0_any_chunk(chunk):
    p = inputs.workload_prefill(0)
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert_close(y, y_ref, 1e-4, f"y chunk {chunk}")
    assert_close(h, h_ref, 1e-4, f"h_out chunk {chunk}")


CASES = [
    # b, L, H, G, P, N, R, io, chunk, h0_std, carry, dist
    (1, 37, 2, 1, 5, 6, 1, "f32", 8, 0.0, False, "tiny"),
    (2, 50, 4, 2, 8, 16, 2, "f32", 16, 0.3, True, "lm"),
    (3, 19, 3, 3, 3, 4, 3, "f32", 4, 0.5, True, "tiny"),
    (1, 70, 2, 1, 16, 32, 4, "bf16", 32, 0.1, True, "lm"),
    (2, 33, 2, 2, 64, 128, 1, "bf16", 16, 0.1, False, "lm"),
    (1, 1, 1, 1, 1, 2, 1, "f32", 1, 0.0, False, "tiny"),
    (1, 65, 1, 1, 64, 128, 2, "f32", 64, 0.2, True, "lm"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_random_shapes(case):
    b, L, H, G, P, N, R, io, chunk, h0s, carry, dist = case
    _flush(f"prefill case {case}")
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist=dist, wid=300 + CASES.index(case), h0_std=h0s, with_carry=carry)
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert_close(y, y_ref, TOL[io], "y")
    assert_close(h, h_ref, TOL[io], "h_out")


def test_empty_sequence_copies_state():
    p = inputs.make_problem(batch=2, seqlen=0, heads=2, groups=1, headdim=4, dstate=4, rank=1, h0_std=1.0)
    y, h = gpu_prefill(p, 16)
    assert torch.equal(h.cpu(), p["h0"])


def run_decode(p, steps_from=0, state=None, device="cuda"):
    """Feed tokens [steps_from, L) of a prefill-shaped problem through m3_decode_step."""
    from mamba_ssm_scan_amd import binding
    d = to_dev(p)
    b, L, H, R, P = d["x"].shape
    G, N = d["B"].shape[2], d["B"].shape[4]
    if state is None:
        state = binding.DecodeState(b, H, G, P, N, R, io_dtype=d["x"].dtype, h0=d.get("h0"),
                                    B_last=d.get("carry_B"), x_last=d.get("carry_x"))
    ys = []
    for t in range(steps_from, L):
        ys.append(state.step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"], d["omega"],
                             d["lam"][:, t].contiguous(), d["B"][:, t].contiguous(), d["C"][:, t].contiguous(),
                             d["D"]))
    torch.cuda.synchronize()
    return torch.stack(ys, 1), state


DCASES = [
    # b, L, H, G, P, N, R, io, carry
    (2, 20, 4, 2, 8, 16, 1, "f32", True),
    (1, 9, 3, 1, 5, 6, 3, "f32", False),
    (2, 12, 3, 1, 64, 128, 1, "f32", True),
    (2, 12, 3, 3, 64, 128, 2, "f32", False),
    (1, 12, 2, 1, 64, 128, 4, "f32", True),
    (3, 10, 4, 1, 64, 128, 1, "bf16", True),
    (2, 10, 4, 2, 64, 128, 4, "bf16", False),
    (2, 10, 3, 3, 64, 128, 2, "bf16", True),
    (1, 8, 4, 1, 64, 128, 4, "bf16", True),
]


@pytest.mark.parametrize("case", DCASES, ids=[str(c) for c in DCASES])
def test_decode_steps(case):
    b, L, H, G, P, N, R, io, carry = case
    _flush(f"decode case {case}")
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist="lm", wid=400 + DCASES.index(case), h0_std=0.1, with_carry=carry)
    y_ref, h_ref = oracle.scan(p)
    y, st = run_decode(p)
    assert st.t == L
    assert_close(y, y_ref, TOL[io], "decode y")
    assert_close(st.h, h_ref, TOL[io], "decode h")


@pytest.mark.parametrize("k", [1, 16, 17, 40])
def test_prefill_then_decode_handoff(k):
    from mamba_ssm_scan_amd import binding
    L = 48
    p = inputs.make_problem(batch=2, seqlen=L, heads=2, groups=1, headdim=8, dstate=16, rank=2, io_dtype="f32",
                            dist="lm", wid=500, h0_std=0.2)
    y_ref, h_ref = oracle.scan(p)
    pre = inputs.slice_tokens(p, 0, k)
    y1, h1 = gpu_prefill(pre, 16)
    d = to_dev(p)
    st = binding.DecodeState(2, 2, 1, 8, 16, 2, io_dtype=torch.float32, h0=h1,
                             B_last=d["B"][:, k - 1].contiguous(), x_last=d["x"][:, k - 1].contiguous(), t0=k)
    y2, st = run_decode(p, steps_from=k, state=st)
    assert st.t == L
    y = np.concatenate([f64(y1), f64(y2)], 1)
    assert_close(y, y_ref, 1e-4, "handoff y")
    assert_close(st.h, h_ref, 1e-4, "handoff h")


def dyadic_problem(L, Q, io, R=1, H=2, P=8, N=16, n0=5):
    """A = 0, omega = 0, dt = 1, lambda = 1/2, one-hot B = C = e_n0, integer impulses.

    Then y_t = sum_{s<t} x_s + 1.5 x_t (rank 0; other ranks zero), exactly.
    """
    p = inputs.make_problem(batch=1, seqlen=L, heads=H, groups=1, headdim=P, dstate=N, rank=R, io_dtype=io,
                            wid=600)
    dt_ = p["x"].dtype
    p["A"] = torch.zeros(H)
    p["omega"] = torch.zeros(H, N // 2)
    p["dt"] = torch.ones(1, L, H)
    p["lam"] = torch.full((1, L, H), 0.5)
    p["D"] = torch.ones(H)
    B = torch.zeros(1, L, 1, R, N)
    B[..., 0, n0] = 1.0
    p["B"] = B.to(dt_)
    p["C"] = B.clone().to(dt_)
    x = torch.zeros(1, L, H, R, P)
    rng = np.random.default_rng(7)
    for k in range(1, L // Q + 1):
        for t in (k * Q - 1, k * Q, k * Q + 1):
            if t < L:
                x[0, t, :, 0, :] = torch.from_numpy(rng.integers(-2, 3, size=(H, P)).astype(np.float32))
    p["x"] = x.to(dt_)
    xs = x[0, :, :, 0, :].double().numpy()
    expect = np.cumsum(xs, 0) - xs + 1.5 * xs
    assert np.abs(expect).max() <= 127.5
    return p, expect


@pytest.mark.parametrize("io,Q", [("f32", 16), ("bf16", 16), ("f32", 7), ("bf16", 64)])
def test_dyadic_exact(io, Q):
    p, expect = dyadic_problem(200, Q, io)
    y_ref, _ = oracle.scan(p)
    assert np.array_equal(y_ref[0, :, :, 0, :], expect)          # the oracle is exact here too
    y, _ = gpu_prefill(p, Q)
    got = f64(y)[0, :, :, 0, :]
    assert np.array_equal(got, expect), np.argwhere(got != expect)[:5]
    assert np.all(f64(y)[0, :, :, 1:, :] == 0)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_coverage_and_guards(io):
    """y and h_out pre-filled with NaN inside guard bands: every element written, no byte outside."""
    from mamba_ssm_scan_amd import binding
    p = to_dev(inputs.make_problem(batch=2, seqlen=45, heads=3, groups=1, headdim=8, dstate=16, rank=2,
                                   io_dtype=io, wid=700, h0_std=0.1))
    guard = 2048
    ny, nh = p["x"].numel(), 2 * 3 * 16 * 8
    ybuf = torch.full((ny + 2 * guard,), float("nan"), dtype=p["x"].dtype, device="cuda")
    hbuf = torch.full((nh + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    y = ybuf[guard:guard + ny].view(p["x"].shape)
    h = hbuf[guard:guard + nh].view(2, 3, 16, 8)
    ypat = ybuf.view(torch.int16 if io == "bf16" else torch.int32).clone()
    hpat = hbuf.view(torch.int32).clone()
    binding.prefill(p["x"], p["dt"], p["A"], p["omega"], p["lam"], p["B"], p["C"], p["D"], 2, 16, p["h0"],
                    y=y, h_out=h)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(h).all()
    yv = ybuf.view(ypat.dtype)
    hv = hbuf.view(torch.int32)
    assert torch.equal(yv[:guard], ypat[:guard]) and torch.equal(yv[-guard:], ypat[-guard:])
    assert torch.equal(hv[:guard], hpat[:guard]) and torch.equal(hv[-guard:], hpat[-guard:])
