"""Seeded random shapes through every entry point, against the fp64 oracles.

Each case draws (b, L, H, G, P, N, R, I/O dtype, chunk, h0, carry, omega / lambda
NULL) from a fixed seed, so the set is the same on every run; the shapes fall on
all three prefill paths (chunked MFMA, token walk, generic), the decode kernels
and the backward. Bars: 1e-4 (fp32 I/O) and 2e-2 (bf16 I/O) max-relative per
(batch, head) slice, as everywhere else.
"""
import random

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bw
from mamba_ssm_scan_amd import binding, inputs
from tests.util import TOL, assert_close, f64, gpu_prefill, to_dev

pytestmark = pytest.mark.gpu


def _draw(seed):
    rnd = random.Random(seed)
    io = rnd.choice(["f32", "bf16", "bf16"])
    fam = rnd.choice(["mfma", "scan", "any"]) if io == "bf16" else "any"
    if fam == "mfma":
        P, N, R = 64, 128, rnd.choice([1, 2, 4])
    elif fam == "scan":
        P, N, R = rnd.choice([16, 32, 48, 64]), rnd.choice([16, 64, 144, 256]), rnd.randint(1, 8)
    else:
        P, N, R = rnd.randint(1, 24), 2 * rnd.randint(1, 12), rnd.randint(1, 5)
    H = rnd.choice([1, 2, 3, 4])
    G = rnd.choice([g for g in (1, 2, H) if H % g == 0])
    return dict(b=rnd.randint(1, 3), L=rnd.randint(1, 150), H=H, G=G, P=P, N=N, R=R, io=io,
                chunk=rnd.choice([8, 16, 33, 64]), h0=rnd.random() < 0.5, carry=rnd.random() < 0.5,
                no_om=rnd.random() < 0.2, no_lam=rnd.random() < 0.2)


def _problem(c, wid):
    p = inputs.make_problem(batch=c["b"], seqlen=c["L"], heads=c["H"], groups=c["G"], headdim=c["P"], dstate=c["N"],
                            rank=c["R"], io_dtype=c["io"], dist="lm", wid=wid, h0_std=0.1 if c["h0"] else 0.0,
                            with_carry=c["carry"])
    q = dict(p)
    if c["no_om"]:
        q["omega"] = torch.zeros_like(p["omega"])
    if c["no_lam"]:
        q["lam"] = torch.ones_like(p["lam"])
    return p, q


SEEDS = list(range(24))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_prefill(seed):
    c = _draw(seed)
    print(f"random prefill {c}", flush=True)
    p, q = _problem(c, 1100 + seed)
    y_ref, h_ref = oracle.scan(q)
    d = to_dev(p)
    y, h = binding.prefill(d["x"], d["dt"], d["A"], None if c["no_om"] else d["omega"],
                           None if c["no_lam"] else d["lam"], d["B"], d["C"], d["D"], c["R"], c["chunk"], d.get("h0"),
                           carry_B=d.get("carry_B"), carry_x=d.get("carry_x"))
    torch.cuda.synchronize()
    assert_close(y, y_ref, TOL[c["io"]], "y")
    assert_close(h, h_ref, TOL[c["io"]], "h_out")


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_decode(seed):
    c = _draw(100 + seed)
    c["L"] = min(c["L"], 12)
    print(f"random decode {c}", flush=True)
    p, q = _problem(c, 1200 + seed)
    y_ref, h_ref = oracle.scan(q)
    d = to_dev(p)
    st = binding.DecodeState(c["b"], c["H"], c["G"], c["P"], c["N"], c["R"], io_dtype=d["x"].dtype, h0=d.get("h0"),
                             B_last=d.get("carry_B"), x_last=d.get("carry_x"))
    ys = [st.step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                  None if c["no_om"] else d["omega"], None if c["no_lam"] else d["lam"][:, t].contiguous(),
                  d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d["D"]) for t in range(c["L"])]
    torch.cuda.synchronize()
    assert_close(torch.stack(ys, 1), y_ref, TOL[c["io"]], "decode y")
    assert_close(st.h, h_ref, TOL[c["io"]], "decode h")


@pytest.mark.parametrize("seed", SEEDS[:12])
def test_random_backward(seed):
    c = _draw(200 + seed)
    c["N"], c["P"], c["R"] = min(c["N"], 128), min(c["P"], 64), min(c["R"], 4)
    if c["io"] == "bf16" and c["P"] % 2:
        c["P"] += 1
    c["L"] = min(c["L"], 70)
    print(f"random backward {c}", flush=True)
    p, q = _problem(c, 1300 + seed)
    g = torch.Generator().manual_seed(seed)
    dt_ = torch.bfloat16 if c["io"] == "bf16" else torch.float32
    dy = torch.randn(p["x"].shape, generator=g).to(dt_)
    dh = torch.randn((c["b"], c["H"], c["N"], c["P"]), generator=g)
    d = to_dev(p)
    out = binding.prefill_backward(d["x"], d["dt"], d["A"], None if c["no_om"] else d["omega"],
                                   None if c["no_lam"] else d["lam"], d["B"], d["C"], d["D"], c["R"], dy.cuda(),
                                   d.get("h0"), dh.cuda(), carry_B=d.get("carry_B"), carry_x=d.get("carry_x"),
                                   want_lambda=not c["no_lam"], want_omega=not c["no_om"])
    torch.cuda.synchronize()
    ref = bw.backward(q, dy, dh)
    tol = TOL[c["io"]]
    for k in ("x", "B", "C", "dt", "A", "D", "h0") + (("lam",) if not c["no_lam"] else ()) + \
            (("omega",) if not c["no_om"] else ()):
        got, r = f64(out[k]), np.asarray(ref[k], np.float64)
        den = np.abs(r).max()
        err = float(np.abs(got - r).max() / den) if den > 0 else float(np.abs(got).max())
        assert np.isfinite(err) and err <= tol, f"d{k}: {err:.2e}"
