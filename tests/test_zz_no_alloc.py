"""m3_prefill_noalloc (the workspace taken from the library's fixed device scratch)
against m3_prefill with a caller workspace and against the oracle, through the C ABI.

Two calls in a row on the same GPU, the second smaller, so the second runs on
scratch the first has left behind; the segmented MIMO path (look-back state in
the scratch), the N 256 row passes (fp32 partial outputs in the scratch) and the
fp32 generic path (running state in the scratch) each take their turn.
"""
import ctypes

import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(q, R, chunk):
    lib = binding.load()
    b, L, H, _, P = q["x"].shape
    G, N = q["B"].shape[2], q["B"].shape[4]
    d = binding.dims(b, L, H, G, P, N)
    code = binding.M3_BF16 if q["x"].dtype == torch.bfloat16 else binding.M3_F32
    y = torch.full_like(q["x"], float("nan"))
    h = torch.full((b, H, N, P), float("nan"), dtype=torch.float32, device="cuda")
    p = binding._ptr
    binding.check(lib.m3_prefill_noalloc(p(q["x"]), p(q["dt"]), p(q["A"]), p(q["omega"]), p(q["lam"]), p(q["B"]),
                                         p(q["C"]), p(q["D"]), R, chunk, p(q.get("h0")), p(y), p(h),
                                         ctypes.byref(d), code, p(q.get("carry_B")), p(q.get("carry_x")),
                                         binding._stream(None)))
    return y, h


# (b, L, H, G, P, N, R, chunk, io, segments, h0_std, carry): each pair of rows runs large then small
CASES = [
    [(1, 1500, 3, 1, 64, 128, 4, 64, "bf16", 4, 0.1, True), (1, 700, 2, 1, 64, 128, 4, 64, "bf16", 2, 0.0, False)],
    [(1, 600, 4, 1, 64, 256, 2, 64, "bf16", 1, 0.1, False), (1, 200, 2, 1, 64, 256, 1, 64, "bf16", 1, 0.0, True)],
    [(2, 300, 2, 1, 8, 16, 1, 16, "f32", 1, 0.1, True), (1, 100, 2, 2, 8, 16, 2, 16, "f32", 1, 0.0, False)],
]


@pytest.mark.parametrize("pair", CASES, ids=["segmented_r4", "n256_row_passes", "generic_f32"])
def test_noalloc_matches_workspace_call(pair, monkeypatch):
    for k, case in enumerate(pair):
        b, L, H, G, P, N, R, chunk, io, nseg, h0s, carry = case
        print(f"noalloc call {k}: {case}", flush=True)
        monkeypatch.setenv("M3_PREFILL_SEGMENTS", str(nseg))
        code = binding.M3_BF16 if io == "bf16" else binding.M3_F32
        plan = binding.plan(binding.dims(b, L, H, G, P, N), R, chunk, code)
        assert plan.segments == nseg and 0 < plan.workspace_bytes <= binding.load().m3_noalloc_scratch_bytes()
        prob = inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R, io_dtype=io,
                                   dist="lm", wid=1300 + 10 * CASES.index(pair) + k, h0_std=h0s, with_carry=carry)
        q = to_dev(prob)
        y_na, h_na = _noalloc(q, R, chunk)
        y_ws, h_ws = binding.prefill(q["x"], q["dt"], q["A"], q["omega"], q["lam"], q["B"], q["C"], q["D"], R, chunk,
                                     q.get("h0"), carry_B=q.get("carry_B"), carry_x=q.get("carry_x"))
        torch.cuda.synchronize()
        y_ref, h_ref = oracle.scan(prob)
        tol = TOL[io]
        assert_close(y_na, y_ref, tol, "noalloc y vs oracle")
        assert_close(h_na, h_ref, tol, "noalloc h_out vs oracle")
        assert_close(y_na, y_ws.double().cpu().numpy(), tol, "noalloc y vs m3_prefill")
        assert_close(h_na, h_ws.double().cpu().numpy(), tol, "noalloc h_out vs m3_prefill")
