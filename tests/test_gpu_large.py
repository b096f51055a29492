"""GPU parity at the larger deployment sizes: state dimension N = 256 and MIMO
ranks R = 6 and 8 (the state-size and rank knobs of "Mamba-3架构技术解析" §4.3
and the MIMO rank of "复值SSM × 广义梯形离散 × MIMO" §2.3).

With bf16 I/O the prefill cases here run the token-walk kernel (state in
registers, rank contractions on MFMA; N, P multiples of 16 up to 256 and 64):
the ranks the chunked MFMA kernels do not take (5 to 8); R 3 runs the chunked R 4
kernel with a zero fourth rank, N 256 at R 1 to 4 the chunked kernels in two row
passes (its full-size case below). fp32 I/O runs the generic chunked kernel,
decode the generic step. The oracle runs the
same problem in fp64; bars are the recurrence's own (1e-4 fp32, 2e-2 bf16 I/O,
max-relative per (batch, head) slice).
"""
import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close, gpu_prefill, to_dev, to_host

pytestmark = pytest.mark.gpu

PCASES = [
    # b, L, H, G, P, N, R, io, chunk
    (1, 150, 2, 1, 48, 256, 5, "bf16", 64),   # N 256, P 48, R 5, a ragged last block
    (2, 70, 2, 1, 64, 128, 8, "bf16", 32),    # R 8
    (1, 90, 3, 3, 64, 256, 6, "bf16", 64),    # N 256 and R 6, one B, C per head
    (2, 41, 4, 2, 64, 128, 7, "bf16", 64),    # R 7; b*H = 8
    (1, 33, 2, 1, 32, 64, 5, "bf16", 64),     # P 32 (two waves idle), N 64, R 5
    (1, 17, 2, 1, 48, 208, 7, "bf16", 64),    # N 208 (13 row tiles), P 48, R 7
    (1, 37, 2, 1, 48, 208, 3, "bf16", 64),    # N 208 with R 3: the chunked R 4 kernel, rank and rows padded
    (3, 1, 2, 1, 32, 256, 6, "bf16", 64),     # one token
    (1, 45, 2, 1, 16, 256, 8, "f32", 16),     # fp32: the generic kernel
]


def _expected_path(io, N, P, R):
    """bf16: the chunked MFMA kernels at R 1-4 and at R 8 with N 128, P 64; the token walk for the rest."""
    if io != "bf16":
        return binding.M3_PATH_GENERIC
    return binding.M3_PATH_MFMA if R <= 4 or (N == 128 and P == 64) else binding.M3_PATH_SCAN


def _path(p, chunk):
    b, L, H, R, P = p["x"].shape
    G, N = p["B"].shape[2], p["B"].shape[4]
    io = binding.M3_BF16 if p["x"].dtype == torch.bfloat16 else binding.M3_F32
    return binding.plan(binding.dims(b, L, H, G, P, N), R, chunk, io).path


@pytest.mark.parametrize("case", PCASES, ids=[str(c) for c in PCASES])
def test_prefill_large_state_and_rank(case):
    b, L, H, G, P, N, R, io, chunk = case
    print(f"prefill large case {case}", flush=True)
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                            dist="lm", wid=1000 + PCASES.index(case), h0_std=0.1, with_carry=True)
    assert _path(p, chunk) == _expected_path(io, N, P, R)
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert_close(y, y_ref, TOL[io], "y")
    assert_close(h, h_ref, TOL[io], "h_out")


R8CASES = [
    # b, L, H, G, R, chunk, h0_std, carry
    (1, 100, 2, 1, 8, 32, 0.1, True),   # four chunks of 32 tokens, a ragged last one
    (2, 77, 3, 3, 8, 64, 0.0, False),   # chunk 64 asked: walked in chunks of 32; one B, C per head
    (1, 45, 2, 2, 8, 16, 0.1, True),    # chunk 16, two groups
    (1, 33, 2, 1, 8, 7, 0.1, False),    # chunk 7
    (2, 5, 2, 1, 8, 32, 0.1, True),     # fewer tokens than a chunk
    (1, 70, 2, 1, 5, 32, 0.1, True),    # R 5, 6, 7: the R 8 kernel with zero ranks
    (2, 41, 2, 2, 6, 64, 0.0, True),
    (1, 90, 3, 1, 7, 32, 0.1, False),
    (1, 130, 2, 1, 3, 64, 0.1, True),   # R 3: the R 4 kernel with a zero fourth rank
    (2, 50, 2, 2, 3, 16, 0.0, False),
]


@pytest.mark.parametrize("case", R8CASES, ids=[str(c) for c in R8CASES])
def test_prefill_r8_chunked(case):
    """R 3 and R 5-8 at N 128, P 64 on the wave-specialised chunked kernels (at R > 4 chunks of at most
    32 tokens), the ranks above R zero."""
    b, L, H, G, R, chunk, h0s, carry = case
    print(f"wave-specialised chunked case {case}", flush=True)
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=64, dstate=128, rank=R, io_dtype="bf16",
                            dist="lm", wid=1100 + R8CASES.index(case), h0_std=h0s, with_carry=carry)
    assert _path(p, chunk) == binding.M3_PATH_MFMA
    plan = binding.plan(binding.dims(b, L, H, G, 64, 128), R, chunk, binding.M3_BF16)
    q = min(chunk, 32) if R > 4 else chunk
    assert plan.n_chunks == (L + q - 1) // q
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


@pytest.mark.parametrize("drop", ["omega", "lam", "both"])
def test_prefill_r8_chunked_special_cases(drop):
    """omega NULL (omega = 0) and lambda NULL (lambda = 1) on the R 8 chunked kernel."""
    print(f"R 8 chunked special case {drop}", flush=True)
    p = inputs.make_problem(batch=1, seqlen=70, heads=2, groups=1, headdim=64, dstate=128, rank=8, io_dtype="bf16",
                            dist="lm", wid=1120, h0_std=0.1, with_carry=True)
    q = dict(p)
    no_om, no_lam = drop in ("omega", "both"), drop in ("lam", "both")
    if no_om:
        q["omega"] = torch.zeros_like(p["omega"])
    if no_lam:
        q["lam"] = torch.ones_like(p["lam"])
    y_ref, h_ref = oracle.scan(q)
    d = to_dev(p)
    y, h = binding.prefill(d["x"], d["dt"], d["A"], None if no_om else d["omega"], None if no_lam else d["lam"],
                           d["B"], d["C"], d["D"], 8, 32, d["h0"], carry_B=d["carry_B"], carry_x=d["carry_x"])
    torch.cuda.synchronize()
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


@pytest.mark.parametrize("drop", ["omega", "lam", "both"])
def test_scan_special_cases(drop):
    """omega NULL (omega = 0) and lambda NULL (lambda = 1) on the token-walk kernel."""
    print(f"scan special case {drop}", flush=True)
    p = inputs.make_problem(batch=2, seqlen=60, heads=2, groups=1, headdim=64, dstate=256, rank=6, io_dtype="bf16",
                            dist="lm", wid=1030, h0_std=0.1, with_carry=True)
    q = dict(p)
    no_om, no_lam = drop in ("omega", "both"), drop in ("lam", "both")
    if no_om:
        q["omega"] = torch.zeros_like(p["omega"])
    if no_lam:
        q["lam"] = torch.ones_like(p["lam"])
    y_ref, h_ref = oracle.scan(q)
    d = to_dev(p)
    y, h = binding.prefill(d["x"], d["dt"], d["A"], None if no_om else d["omega"], None if no_lam else d["lam"],
                           d["B"], d["C"], d["D"], 6, 64, d["h0"], carry_B=d["carry_B"], carry_x=d["carry_x"])
    torch.cuda.synchronize()
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


@pytest.mark.parametrize("wid,dstate,rank", [(1, 256, None), (2, None, 8)])
def test_workload_shapes_larger_state_and_rank(wid, dstate, rank):
    """Workload 1's shape with N 256, workload 2's with R 8 (b 4, L 2048, H 64): the oracle runs every walk."""
    w = inputs.WORKLOADS[wid]
    N, R = dstate or w.dstate, rank or w.rank
    print(f"workload {wid} shape with N {N}, R {R}", flush=True)
    p = inputs.make_problem(batch=w.batch, seqlen=w.seqlen, heads=w.heads, groups=1, headdim=w.headdim, dstate=N,
                            rank=R, io_dtype=w.io_dtype, dist=w.dist, wid=wid, device="cuda")
    assert _path(p, w.chunk) == binding.M3_PATH_MFMA  # R 8 at N 128, P 64: the wave-specialised chunked kernel
    y, h = binding.prefill(p["x"], p["dt"], p["A"], p["omega"], p["lam"], p["B"], p["C"], p["D"], R, w.chunk)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.scan(to_host(p))
    assert_close(y, y_ref, TOL["bf16"], "y, all heads and batches")
    assert_close(h, h_ref, TOL["bf16"], "h_out, all heads and batches")


DCASES = [
    # b, L, H, G, P, N, R, io
    (2, 8, 2, 1, 64, 256, 1, "bf16"),   # the float4 row kernel at N 256
    (2, 8, 2, 1, 64, 128, 8, "bf16"),   # the MFMA decode kernel at R 8 (two k groups of ranks)
    (1, 6, 3, 1, 64, 64, 8, "bf16"),
    (1, 6, 3, 3, 64, 256, 6, "f32"),
    # the float4 row kernel at the other (N, P) it is built for (bf16 I/O, R 1, 2, 4)
    (2, 6, 2, 1, 32, 64, 1, "bf16"),
    (1, 6, 3, 1, 64, 64, 4, "bf16"),   # (P 64, N 64, R 4: the merged-input MFMA kernel)
    (2, 5, 2, 2, 128, 64, 2, "bf16"),
    (1, 6, 2, 1, 32, 128, 4, "bf16"),
    (2, 6, 2, 1, 128, 128, 1, "bf16"),
    (1, 6, 2, 1, 32, 256, 2, "bf16"),
    (1, 5, 4, 2, 64, 256, 4, "bf16"),
    (1, 6, 2, 1, 128, 256, 1, "bf16"),
    (2, 6, 2, 1, 64, 128, 3, "bf16"),   # R 3: the merged-input MFMA kernel with a zero rank slot
    # the merged-input MFMA kernel at R 2, 3 and N 64, 128, with groups
    (2, 6, 4, 2, 64, 64, 2, "bf16"),
    (1, 6, 2, 1, 64, 64, 3, "bf16"),
    (2, 6, 4, 2, 64, 128, 2, "bf16"),
    (1, 7, 4, 2, 64, 128, 4, "bf16"),
    # R 3 and R 8 on the row kernel
    (1, 5, 2, 1, 128, 256, 3, "bf16"),
    (2, 6, 2, 2, 32, 64, 8, "bf16"),
    (1, 6, 2, 1, 128, 128, 8, "bf16"),  # R 8 past the row kernel's LDS: the generic step
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
