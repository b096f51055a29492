"""The C entry points under HIP graph capture (torch.cuda.graph on the caller's stream).

Every launch path of libm3 is capturable: kernels only, no allocation, no
memset (the prefill's look-back counters are cleared by a fill kernel), no
host synchronisation. Each test runs the calls eagerly, captures the same
calls into a graph, then replays the graph several times with eager torch work
and synchronisations in between, and requires every replay to reproduce the
eager outputs: bit for bit where the kernels are deterministic (decode, the
prologue), and to fp32 rounding where sequence segments combine their
predecessors' states in an order set by which one finished first (the
look-back of the segmented prefill).
"""
import pytest
import torch

import oracle
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close

pytestmark = pytest.mark.gpu


def _noise():
    # unrelated eager work between replays
    a = torch.randn(1 << 20, device="cuda")
    (a * 2 + 1).sum().item()


def test_prologue_and_segmented_prefill_replay():
    print("case prologue + R 4 prefill with 4 segments under capture", flush=True)
    b, L, H, G, P, N, R = 1, 2048, 8, 1, 64, 128, 4
    raw = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
           for k, v in inputs.prologue_inputs(tokens=(b, L), heads=H, groups=G, rank=R, dstate=N,
                                              io_dtype="bf16", wid=400).items()}
    p = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
         for k, v in inputs.make_problem(batch=b, seqlen=L, heads=H, groups=G, headdim=P, dstate=N, rank=R,
                                         io_dtype="bf16", dist="lm", wid=401).items()}
    plan = binding.plan(binding.dims(b, L, H, G, P, N), R, 64, binding.M3_BF16)
    assert plan.segments > 1, "the case should exercise the look-back counters"
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
    Bn, Cn = torch.empty_like(raw["B_raw"]), torch.empty_like(raw["C_raw"])
    dt, lam = torch.empty_like(raw["dt_raw"]), torch.empty_like(raw["lambda_raw"])
    y = torch.empty_like(p["x"])
    h = torch.empty((b, H, N, P), dtype=torch.float32, device="cuda")

    def calls():
        binding.prologue(raw["B_raw"], raw["C_raw"], B_weight=raw["B_weight"], B_bias=raw["B_bias"],
                         C_weight=raw["C_weight"], C_bias=raw["C_bias"], eps=1e-6, dt_raw=raw["dt_raw"],
                         dt_bias=raw["dt_bias"], lambda_raw=raw["lambda_raw"], B=Bn, C=Cn, dt=dt, lam=lam)
        binding.prefill(p["x"], dt, p["A"], p["omega"], lam, Bn, Cn, p["D"], R, 64, y=y, h_out=h, workspace=ws)

    calls()
    torch.cuda.synchronize()
    y_ref, h_ref = y.clone(), h.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the side stream, as capture wants
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    B_ref, dt_ref = Bn.clone(), dt.clone()
    for rep in range(3):
        y.zero_()
        h.fill_(float("nan"))
        Bn.zero_()
        dt.zero_()
        _noise()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Bn, B_ref) and torch.equal(dt, dt_ref), f"replay {rep}: prologue differs"
        # segments wait for their predecessor's inclusive state only: every replay
        # combines the same values in the same order, so the outputs are bit-identical
        ey = ((y.float() - y_ref.float()).abs().max() / y_ref.float().abs().max()).item()
        eh = ((h - h_ref).abs().max() / h_ref.abs().max()).item()
        print(f"  replay {rep}: y {ey:.2e}, h_out {eh:.2e}", flush=True)
        assert torch.equal(y, y_ref) and torch.equal(h, h_ref), f"replay {rep}: y {ey:.2e}, h_out {eh:.2e}"


def test_decode_steps_replay():
    print("case 8 decode steps (R 4, b 4) under capture", flush=True)
    b, H, G, P, N, R, steps = 4, 8, 1, 64, 128, 4, 8
    di = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
          for k, v in inputs.decode_inputs(3, steps, device="cpu", rank=R, batch=b).items()}
    Hs = slice(0, H)
    x = di["x"][:, :, Hs].contiguous()
    dtv, lamv = di["dt"][:, :, Hs].contiguous(), di["lam"][:, :, Hs].contiguous()
    A, om, D = di["A"][Hs].contiguous(), di["omega"][Hs].contiguous(), di["D"][Hs].contiguous()
    h0 = di["h0"][:, Hs].contiguous()
    ys = torch.empty_like(x)
    st = binding.DecodeState(b, H, G, P, N, R, io_dtype=torch.bfloat16, h0=h0)
    h_init, cB_init, cx_init = st.h.clone(), st.carry_B.clone(), st.carry_x.clone()

    def calls():
        for t in range(steps):
            st.step(x[t], dtv[t], A, om, lamv[t], di["B"][t], di["C"][t], D, y_t=ys[t])

    def reset():
        st.h.copy_(h_init)
        st.carry_B.copy_(cB_init)
        st.carry_x.copy_(cx_init)

    calls()
    torch.cuda.synchronize()
    y_ref, h_ref = ys.clone(), st.h.clone()
    t_after = st.t
    reset()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        reset()
        ys.zero_()
        _noise()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, y_ref), f"replay {rep}: y differs"
        assert torch.equal(st.h, h_ref), f"replay {rep}: state differs"
    assert st.t == t_after + steps  # the host counter advanced once, at capture


@pytest.mark.parametrize("R,G", [(1, 1), (4, 1), (1, 2), (4, 2)])
def test_decode_odd_graph_replays_continue(R, G):
    """A captured graph of an odd number of steps (5), replayed twice back to back
    with nothing reset in between, continues the sequence: the 10 outputs and the
    final state equal the oracle over the 5 tokens fed twice. Each step reads
    only device buffers (B_prev from the slot each head's parity word names, x_prev
    from the head's own carry), so the replays do not depend on how many steps
    were captured; G 2 puts two heads in each group."""
    print(f"case odd graph (5 steps, R {R}, G {G}) replayed twice", flush=True)
    b, H, P, N, steps = 2, 4, 64, 128, 5
    di = {k: (v.cuda() if isinstance(v, torch.Tensor) else v)
          for k, v in inputs.decode_inputs(3, steps, device="cpu", rank=R, batch=b, groups=G).items()}
    Hs = slice(0, H)
    x = di["x"][:, :, Hs].contiguous()
    dtv, lamv = di["dt"][:, :, Hs].contiguous(), di["lam"][:, :, Hs].contiguous()
    A, om, D = di["A"][Hs].contiguous(), di["omega"][Hs].contiguous(), di["D"][Hs].contiguous()
    h0 = di["h0"][:, Hs].contiguous()
    Bv, Cv = di["B"].contiguous(), di["C"].contiguous()
    ys = torch.empty_like(x)
    st = binding.DecodeState(b, H, G, P, N, R, io_dtype=torch.bfloat16, h0=h0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(steps):
            st.step(x[t], dtv[t], A, om, lamv[t], Bv[t], Cv[t], D, y_t=ys[t])
    outs = []
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        outs.append(ys.clone())
    # oracle over the 10 tokens (the 5 fed twice), batch-major
    twice = lambda t: torch.cat([t, t], 0).transpose(0, 1).contiguous().cpu()
    prob = {"x": twice(x), "B": twice(Bv), "C": twice(Cv), "dt": twice(dtv), "lam": twice(lamv),
            "A": A.cpu(), "omega": om.cpu(), "D": D.cpu(), "h0": h0.cpu(), "R": R, "io_dtype": "bf16",
            "carry_B": None, "carry_x": None}
    y_ref, h_ref = oracle.scan(prob)
    y = torch.cat(outs, 0).transpose(0, 1).contiguous()
    assert_close(y, y_ref, TOL["bf16"], "y over both replays")
    assert_close(st.h, h_ref, TOL["bf16"], "state after both replays")
