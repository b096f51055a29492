"""GPU parity of the bf16-MFMA chunked prefill: N = 128, P = 64 (below zero-padded, above in row / column passes), R in {1, 2, 4}.

Small cases cover every chunk size class, ragged tails, groups, initial state and
carry; full-size workloads compare every (batch, head) walk with the oracle
(the decode workload: every head of 3 of its 128 sequences).
Tolerance: max-relative error per (batch, head) slice <= 2e-2 (bf16 I/O, fp32 state).
"""
import numpy as np
import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.test_gpu_generic import dyadic_problem, run_decode
from tests.util import TOL, assert_close, f64, gpu_prefill, to_dev, to_host

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _path(b, L, H, G, R, chunk):
    return binding.plan(binding.dims(b, L, H, G, 64, 128), R, chunk, binding.M3_BF16).path


CASES = [
    # b, L, H, G, R, chunk, h0_std, carry
    (1, 64, 2, 1, 1, 64, 0.0, False),
    (2, 200, 3, 1, 1, 64, 0.1, True),
    (1, 130, 4, 4, 1, 64, 0.1, False),
    (1, 100, 2, 1, 2, 64, 0.0, True),
    (2, 150, 2, 2, 2, 32, 0.1, False),
    (1, 257, 2, 1, 4, 64, 0.1, True),
    (1, 90, 3, 3, 4, 64, 0.0, False),
    (1, 77, 2, 1, 4, 16, 0.1, False),
    (1, 50, 2, 1, 1, 7, 0.1, True),
    (1, 41, 2, 1, 4, 1, 0.0, True),
    (1, 1, 2, 1, 4, 64, 0.1, True),
    (1, 65, 1, 1, 1, 33, 0.1, False),
    (1, 130, 2, 1, 3, 64, 0.1, True),   # R 3: the R 4 kernel with a zero fourth rank
    (2, 97, 3, 3, 3, 16, 0.0, True),
    (1, 1100, 2, 1, 3, 64, 0.1, True),  # R 3 with sequence segments (look-back, output correction)
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_mfma_small(case):
    b, L, H, G, R, chunk, h0s, carry = case
    assert _path(b, L, H, G, R, chunk) == binding.M3_PATH_MFMA
    _flush(f"mfma case {case}")
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=64, dstate=128, rank=R, io_dtype="bf16",
                            dist="lm", wid=800 + CASES.index(case), h0_std=h0s, with_carry=carry)
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


PADDED = [
    # b, L, H, G, N, R, chunk, h0_std, carry
    (1, 130, 2, 1, 64, 1, 64, 0.1, True),
    (2, 97, 2, 2, 32, 1, 33, 0.0, False),
    (1, 200, 3, 1, 8, 1, 64, 0.1, True),
    (1, 150, 2, 1, 64, 2, 64, 0.1, True),
    (1, 257, 2, 2, 120, 4, 64, 0.1, True),
    (1, 70, 2, 1, 16, 4, 16, 0.0, True),
    (1, 1100, 2, 1, 64, 4, 64, 0.1, True),  # two sequence segments (look-back) on the padded rows
]


@pytest.mark.parametrize("case", PADDED, ids=[str(c) for c in PADDED])
def test_mfma_padded_state(case):
    """N below 128 runs zero-padded to 128 rows inside the kernels: same results as the oracle at N."""
    b, L, H, G, N, R, chunk, h0s, carry = case
    plan = binding.plan(binding.dims(b, L, H, G, 64, N), R, chunk, binding.M3_BF16)
    assert plan.path == binding.M3_PATH_MFMA
    if L == 1100:
        assert plan.segments == 2
    _flush(f"mfma padded-state case {case}")
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=64, dstate=N, rank=R, io_dtype="bf16",
                            dist="lm", wid=880 + PADDED.index(case), h0_std=h0s, with_carry=carry)
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert tuple(h.shape) == (b, H, N, 64)
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


PASSES = [
    # b, L, H, G, N, R, chunk, h0_std, carry
    (1, 150, 2, 1, 256, 1, 64, 0.1, True),
    (2, 70, 2, 2, 200, 1, 33, 0.0, True),    # last pass zero-padded (72 rows)
    (1, 100, 2, 1, 384, 2, 64, 0.1, True),   # three passes: a middle one
    (1, 90, 3, 3, 256, 4, 64, 0.1, True),
    (1, 77, 2, 1, 136, 4, 16, 0.0, True),    # last pass 8 rows
    (1, 40, 2, 1, 512, 4, 64, 0.1, False),   # four passes
    (1, 1100, 2, 1, 256, 4, 64, 0.1, True),  # few walks, long: one segment (no look-back across passes)
]


@pytest.mark.parametrize("case", PASSES, ids=[str(c) for c in PASSES])
def test_mfma_row_passes(case):
    """N above 128 in passes of 128 rows (outputs summed in fp32 in the workspace): oracle at N."""
    b, L, H, G, N, R, chunk, h0s, carry = case
    plan = binding.plan(binding.dims(b, L, H, G, 64, N), R, chunk, binding.M3_BF16)
    assert plan.path == binding.M3_PATH_MFMA and plan.segments == 1
    assert plan.workspace_bytes >= b * L * H * R * 64 * 4
    _flush(f"mfma row-pass case {case}")
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=64, dstate=N, rank=R, io_dtype="bf16",
                            dist="lm", wid=890 + PASSES.index(case), h0_std=h0s, with_carry=carry)
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert tuple(h.shape) == (b, H, N, 64)
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


COLS = [
    # b, L, H, G, P, N, R, chunk, h0_std, carry
    (1, 130, 2, 1, 32, 128, 1, 64, 0.1, True),
    (2, 77, 2, 2, 8, 64, 1, 33, 0.0, True),
    (1, 100, 3, 1, 48, 128, 2, 64, 0.1, True),
    (1, 150, 2, 1, 128, 128, 1, 64, 0.1, True),    # two column passes
    (1, 90, 2, 2, 200, 256, 4, 64, 0.1, True),     # 4 column x 2 row passes, last column pass 8 wide
    (1, 70, 2, 1, 96, 64, 4, 16, 0.0, True),
    (1, 1100, 2, 1, 32, 64, 4, 64, 0.1, True),     # one pass, padded rows and columns, two segments
]


@pytest.mark.parametrize("case", COLS, ids=[str(c) for c in COLS])
def test_mfma_column_passes(case):
    """P other than 64: below zero-padded, above in passes of 64 columns (each its own problem)."""
    b, L, H, G, P, N, R, chunk, h0s, carry = case
    plan = binding.plan(binding.dims(b, L, H, G, P, N), R, chunk, binding.M3_BF16)
    assert plan.path == binding.M3_PATH_MFMA
    if L == 1100:
        assert plan.segments == 2
    _flush(f"mfma column-pass case {case}")
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype="bf16",
                            dist="lm", wid=970 + COLS.index(case), h0_std=h0s, with_carry=carry)
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, chunk)
    assert tuple(h.shape) == (b, H, N, P)
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


@pytest.mark.parametrize("R,Q", [(1, 64), (4, 64), (2, 16), (4, 5)])
def test_mfma_dyadic_exact(R, Q):
    """Exact index bookkeeping: integer impulses around chunk edges, exact arithmetic."""
    p, expect = dyadic_problem(300, Q, "bf16", R=R, H=2, P=64, N=128, n0=77)
    assert _path(1, 300, 2, 1, R, Q) == binding.M3_PATH_MFMA
    y, _ = gpu_prefill(p, Q)
    got = f64(y)
    assert np.array_equal(got[0, :, :, 0, :], expect), np.argwhere(got[0, :, :, 0, :] != expect)[:5]
    assert np.all(got[0, :, :, 1:, :] == 0)


@pytest.mark.parametrize("R", [1, 4])
def test_mfma_coverage_and_guards(R):
    p = to_dev(inputs.make_problem(batch=2, seqlen=99, heads=3, groups=1, headdim=64, dstate=128, rank=R,
                                   io_dtype="bf16", wid=850, h0_std=0.1))
    guard = 4096
    ny, nh = p["x"].numel(), 2 * 3 * 128 * 64
    ybuf = torch.full((ny + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    hbuf = torch.full((nh + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    y = ybuf[guard:guard + ny].view(p["x"].shape)
    h = hbuf[guard:guard + nh].view(2, 3, 128, 64)
    ypat, hpat = ybuf.view(torch.int16).clone(), hbuf.view(torch.int32).clone()
    binding.prefill(p["x"], p["dt"], p["A"], p["omega"], p["lam"], p["B"], p["C"], p["D"], R, 64, p["h0"],
                    y=y, h_out=h)
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(h).all()
    yv, hv = ybuf.view(torch.int16), hbuf.view(torch.int32)
    assert torch.equal(yv[:guard], ypat[:guard]) and torch.equal(yv[-guard:], ypat[-guard:])
    assert torch.equal(hv[:guard], hpat[:guard]) and torch.equal(hv[-guard:], hpat[-guard:])


def test_mfma_chunk_sweep_agrees():
    """Different chunk sizes give the same result within the bf16 tolerance of the oracle."""
    p = inputs.make_problem(batch=1, seqlen=181, heads=2, groups=1, headdim=64, dstate=128, rank=2,
                            io_dtype="bf16", dist="lm", wid=860, h0_std=0.1, with_carry=True)
    y_ref, h_ref = oracle.scan(p)
    for Q in (1, 2, 3, 8, 13, 31, 32, 63, 64):
        y, h = gpu_prefill(p, Q)
        assert_close(y, y_ref, TOL["bf16"], f"y chunk {Q}")
        assert_close(h, h_ref, TOL["bf16"], f"h chunk {Q}")


@pytest.mark.parametrize("groups", [1, 64])
@pytest.mark.parametrize("wid", [1, 2])
def test_workload_full_size(wid, groups):
    """Workloads 1 (R=1) and 2 (R=4) at full size, chunk 64, in the launch bench.py
    times; the oracle runs every (batch, head) walk (4 x 64 x 2048 tokens).

    groups 1 is the primary reading (B, C shared by all heads); groups 64 gives
    every head its own B, C (the secondary reading, 64x the B/C bytes).
    """
    _flush(f"workload {wid} full size, G {groups}")
    p = inputs.workload_prefill(wid, device="cuda", groups=groups)
    w = inputs.WORKLOADS[wid]
    assert _path(w.batch, w.seqlen, w.heads, groups, w.rank, w.chunk) == binding.M3_PATH_MFMA
    y, h = binding.prefill(p["x"], p["dt"], p["A"], p["omega"], p["lam"], p["B"], p["C"], p["D"], w.rank, w.chunk)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.scan(to_host(p))
    assert_close(y, y_ref, TOL["bf16"], "y, all heads and batches")
    assert_close(h, h_ref, TOL["bf16"], "h_out, all heads and batches")


def test_workload4_prefill_then_decode():
    """Workload 4: prefill of 32768 tokens (R=4), then 256 decode steps, against one
    33024-token oracle run of every head."""
    w = inputs.WORKLOADS[4]
    _flush("workload 4: long prefill + decode handoff")
    p = inputs.long_sequence(4, device="cuda")
    L = w.seqlen
    pre = inputs.slice_tokens(p, 0, L)
    y1, h1 = binding.prefill(pre["x"], pre["dt"], pre["A"], pre["omega"], pre["lam"], pre["B"], pre["C"], pre["D"],
                             w.rank, w.chunk)
    st = binding.DecodeState(1, w.heads, 1, w.headdim, w.dstate, w.rank, io_dtype=torch.bfloat16, h0=h1,
                             B_last=p["B"][:, L - 1].contiguous(), x_last=p["x"][:, L - 1].contiguous(), t0=L)
    y2, st = run_decode(p, steps_from=L, state=st)
    assert st.t == L + w.decode_steps
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.scan(to_host(p))
    assert_close(y1, y_ref[:, :L], TOL["bf16"], "y prefill, all heads")
    assert_close(y2, y_ref[:, L:], TOL["bf16"], "y decode, all heads")
    assert_close(st.h, h_ref, TOL["bf16"], "final state, all heads")


def test_mfma_long_siso_absolute_angle():
    """R=1, 32768 tokens (512 chunks): B and C are turned by the absolute angle
    omega * (total step), which reaches thousands of radians; the per-chunk base
    angle must keep the rotation accurate to the end (y of late tokens, h_out)."""
    _flush("long SISO sequence, 32768 tokens")
    p = inputs.make_problem(batch=1, seqlen=32768, heads=2, groups=1, headdim=64, dstate=128, rank=1,
                            io_dtype="bf16", dist="lm", wid=870, h0_std=0.1, with_carry=True)
    assert _path(1, 32768, 2, 1, 1, 64) == binding.M3_PATH_MFMA
    y_ref, h_ref = oracle.scan(p)
    y, h = gpu_prefill(p, 64)
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(y[:, -2048:], y_ref[:, -2048:], TOL["bf16"], "y, last 2048 tokens")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


@pytest.mark.parametrize("R", [1, 4])
def test_workload3_decode_full_size(R):
    """Workload 3 at full size, as bench.py runs it: b 128, H 64, 1024 decode steps,
    bf16 I/O from an fp32 state h0 ~ N(0, 0.1); the oracle runs every head of
    3 of the 128 sequences over all 1024 steps."""
    w = inputs.WORKLOADS[3]
    steps = 1024
    _flush(f"workload 3 full size, R={R}")
    di = inputs.decode_inputs(3, steps, device="cuda", rank=R)
    st = binding.DecodeState(w.batch, w.heads, 1, w.headdim, w.dstate, R, io_dtype=torch.bfloat16, h0=di["h0"])
    ys = [st.step(di["x"][t], di["dt"][t], di["A"], di["omega"], di["lam"][t], di["B"][t], di["C"][t], di["D"])
          for t in range(steps)]
    torch.cuda.synchronize()
    bs = [0, 77, 127]
    bi = torch.tensor(bs, device="cuda")
    sel = lambda t: t.index_select(1, bi).transpose(0, 1)      # [steps][b]... -> [b'][steps]...
    sub = {"x": sel(di["x"]), "B": sel(di["B"]), "C": sel(di["C"]), "dt": sel(di["dt"]), "lam": sel(di["lam"]),
           "A": di["A"], "omega": di["omega"], "D": di["D"], "h0": di["h0"].index_select(0, bi), "R": R,
           "io_dtype": "bf16", "carry_B": None, "carry_x": None}
    y_ref, h_ref = oracle.scan(to_host({k: (v.contiguous() if isinstance(v, torch.Tensor) else v)
                                        for k, v in sub.items()}))
    y = torch.stack(ys, 1).index_select(0, bi)
    assert_close(y, y_ref, TOL["bf16"], "y (1024 steps), all heads of 3 sequences")
    assert_close(st.h.index_select(0, bi), h_ref, TOL["bf16"], "state after 1024 steps, all heads of 3 sequences")
