"""Sequence-segment parallelism (look-back + correction) of the MFMA prefill (at N 128,
P 64 on the wave-specialised kernel, elsewhere on the single-role one).

Segments are forced with M3_PREFILL_SEGMENTS on small problems; every case is
compared with the oracle, and the workspace's look-back error flag must stay 0
(m3_prefill_check). A spin limit of 0 (M3_LOOKBACK_SPIN_LIMIT) makes every wait
give up at once, and m3_prefill_check must then report it.
"""
import ctypes

import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # b, L, H, G, R, chunk, nseg, h0_std, carry
    (1, 640, 2, 1, 4, 64, 2, 0.0, False),
    (1, 700, 3, 1, 4, 64, 3, 0.1, True),
    (2, 1000, 2, 2, 2, 64, 5, 0.1, False),
    (1, 333, 2, 1, 4, 16, 4, 0.1, True),
    (1, 257, 1, 1, 2, 32, 7, 0.0, False),
    (1, 520, 2, 1, 3, 64, 3, 0.1, True),   # R 3: zero fourth rank, with segments
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_segments_match_oracle(case, monkeypatch):
    b, L, H, G, R, chunk, nseg, h0s, carry = case
    print(f"segments case {case}", flush=True)
    monkeypatch.setenv("M3_PREFILL_SEGMENTS", str(nseg))
    d = binding.dims(b, L, H, G, 64, 128)
    plan = binding.plan(d, R, chunk, binding.M3_BF16)
    assert plan.path == binding.M3_PATH_MFMA and plan.segments > 1
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=64, dstate=128, rank=R, io_dtype="bf16",
                            dist="lm", wid=1100 + CASES.index(case), h0_std=h0s, with_carry=carry)
    # a slow decay on one head keeps the correction running across many chunks
    p["A"][0] = -0.02
    y_ref, h_ref = oracle.scan(p)
    q = to_dev(p)
    ws = torch.full((plan.workspace_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    y, h = binding.prefill(q["x"], q["dt"], q["A"], q["omega"], q["lam"], q["B"], q["C"], q["D"], R, chunk, q.get("h0"),
                           carry_B=q.get("carry_B"), carry_x=q.get("carry_x"), workspace=ws)
    torch.cuda.synchronize()
    ctrl = ws[:8].view(torch.int32).cpu()
    assert int(ctrl[0]) == b * H * plan.segments     # every workgroup took one ticket
    assert int(ctrl[1]) == 0                          # no look-back wait ran out
    assert binding.load().m3_prefill_check(ctypes.byref(d), R, chunk, binding.M3_BF16, binding._ptr(ws),
                                           plan.workspace_bytes, binding._stream(None)) == 0
    assert_close(y, y_ref, TOL["bf16"], "y")
    assert_close(h, h_ref, TOL["bf16"], "h_out")


def test_segments_repeat_with_one_workspace(monkeypatch):
    """Back-to-back calls reuse the workspace: flags are cleared on the stream each call."""
    monkeypatch.setenv("M3_PREFILL_SEGMENTS", "3")
    p = to_dev(inputs.make_problem(batch=1, seqlen=600, heads=2, groups=1, headdim=64, dstate=128, rank=4,
                                   io_dtype="bf16", dist="lm", wid=1150))
    plan = binding.plan(binding.dims(1, 600, 2, 1, 64, 128), 4, 64, binding.M3_BF16)
    ws = torch.empty((plan.workspace_bytes,), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        y, h = binding.prefill(p["x"], p["dt"], p["A"], p["omega"], p["lam"], p["B"], p["C"], p["D"], 4, 64,
                               workspace=ws)
        outs.append((y.clone(), h.clone()))
    torch.cuda.synchronize()
    for y, h in outs[1:]:
        assert torch.equal(y, outs[0][0]) and torch.equal(h, outs[0][1])


def test_lookback_give_up_is_reported(monkeypatch):
    """With the spin limit forced to 0 every look-back wait gives up at once (the kernels
    all finish; the outputs are not valid): m3_prefill_check reports M3_ELOOKBACK for
    that workspace, and for the no-alloc scratch; the next call with the normal limit
    clears the flag and matches the oracle again."""
    lib = binding.load()
    b, L, H, G, R, chunk = 1, 700, 2, 1, 4, 64
    monkeypatch.setenv("M3_PREFILL_SEGMENTS", "3")
    d = binding.dims(b, L, H, G, 64, 128)
    plan = binding.plan(d, R, chunk, binding.M3_BF16)
    assert plan.segments == 3
    p = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=64, dstate=128, rank=R, io_dtype="bf16",
                            dist="lm", wid=1170)
    q = to_dev(p)
    ws = torch.zeros((plan.workspace_bytes,), dtype=torch.uint8, device="cuda")
    sh = binding._stream(None)

    def run(limit):
        monkeypatch.setenv("M3_LOOKBACK_SPIN_LIMIT", str(limit))
        print(f"  segmented prefill with spin limit {limit}", flush=True)
        return binding.prefill(q["x"], q["dt"], q["A"], q["omega"], q["lam"], q["B"], q["C"], q["D"], R, chunk,
                               workspace=ws)

    run(0)
    assert lib.m3_prefill_check(ctypes.byref(d), R, chunk, binding.M3_BF16, binding._ptr(ws), plan.workspace_bytes,
                                sh) == 8
    assert "gave up" in lib.m3_last_error().decode()
    y, h = run(1 << 24)
    assert lib.m3_prefill_check(ctypes.byref(d), R, chunk, binding.M3_BF16, binding._ptr(ws), plan.workspace_bytes,
                                sh) == 0
    y_ref, h_ref = oracle.scan(p)
    assert_close(y, y_ref, TOL["bf16"], "y after the flag cleared")
    # the same through the no-alloc entry point's scratch (NULL workspace)
    monkeypatch.setenv("M3_LOOKBACK_SPIN_LIMIT", "0")
    y2 = torch.empty_like(q["x"])
    binding.check(lib.m3_prefill_noalloc(binding._ptr(q["x"]), binding._ptr(q["dt"]), binding._ptr(q["A"]),
                                         binding._ptr(q["omega"]), binding._ptr(q["lam"]), binding._ptr(q["B"]),
                                         binding._ptr(q["C"]), binding._ptr(q["D"]), R, chunk, None, binding._ptr(y2),
                                         None, ctypes.byref(d), binding.M3_BF16, None, None, sh))
    assert lib.m3_prefill_check(ctypes.byref(d), R, chunk, binding.M3_BF16, None, 0, sh) == 8
