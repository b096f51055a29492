"""Seeded synthetic inputs for the Mamba-3 SSM recurrence.

This module only draws random tensors with the shapes and distributions of the
five workloads below; it holds none of the recurrence's arithmetic. Both the
HIP path and the CPU oracle read the tensors it returns (the oracle after a
copy to host memory), so the two sides always see identical bytes.

Shapes (row-major, contiguous):
  x, y       [b][L][H][R][P]   token inputs / outputs (bf16 or fp32)
  B, C       [b][L][G][R][N]   input / output projections (bf16 or fp32)
  dt, lam    [b][L][H]         step size Delta and trapezoid weight lambda (fp32)
  A, D       [H]               decay rate (A < 0) and skip weight (fp32)
  omega      [H][N/2]          rotation frequency per head and state pair (fp32)
  h0         [b][H][N][P]      initial state (fp32), or None for a zero state
  carry_B    [b][G][R][N], carry_x [b][H][R][P]: the token before the first one
             (None means no previous token)

Distributions (N(mu, s): s is the standard deviation):
  "tiny"  : x, B, C ~ N(0,1), B and C L2-normalised over N per (token, group,
            rank); Delta = softplus(N(-1, 0.5)); A = -exp(U(ln 0.5, ln 4));
            omega ~ U(0, pi); lambda = sigmoid(N(0,1)); D = 1.
  "lm"    : as "tiny" but A = -exp(U(ln 0.5, ln 16)), B and C RMS-normalised
            over N, D ~ N(1, 0.1).
The normalisation is applied in fp32 before rounding to the I/O dtype
(round-to-nearest-even for bf16, which is what torch's conversion does).

Seeds: one torch generator per tensor, seeded from
numpy SeedSequence([20261203, workload_id, tensor_id, step]).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

ROOT_SEED = 20261203

# tensor ids used in the seed sequence
_TID = {"x": 1, "B": 2, "C": 3, "dt": 4, "lam": 5, "A": 6, "omega": 7, "D": 8,
        "h0": 9, "carry_B": 10, "carry_x": 11, "B_raw": 12, "C_raw": 13, "B_weight": 14, "B_bias": 15,
        "C_weight": 16, "C_bias": 17, "dt_raw": 18, "dt_bias": 19, "lambda_raw": 20, "row_scale": 21,
        "u": 22, "W_x": 23, "W_z": 24, "W_B": 25, "W_C": 26, "W_dt": 27, "W_lambda": 28, "W_out": 29}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named workload: shapes, chunk, I/O dtype, distribution family."""
    wid: int
    name: str
    batch: int
    heads: int
    headdim: int      # P
    dstate: int       # N
    rank: int         # R
    seqlen: int       # L (prefill tokens; 0 for a pure decode loop)
    chunk: int        # Q
    io_dtype: str     # "f32" or "bf16"
    dist: str         # "tiny" or "lm"
    decode_steps: int = 0
    h0_std: float = 0.0


WORKLOADS = {
    0: Workload(0, "tiny_siso_fp32_b1_h2_p8_n16_l128_q16", 1, 2, 8, 16, 1, 128, 16, "f32", "tiny"),
    1: Workload(1, "siso_prefill_b4_h64_p64_n128_l2048_q64", 4, 64, 64, 128, 1, 2048, 64, "bf16", "lm"),
    2: Workload(2, "mimo_r4_prefill_b4_h64_p64_n128_l2048_q64", 4, 64, 64, 128, 4, 2048, 64, "bf16", "lm"),
    3: Workload(3, "decode_b128_h64_p64_n128_1024_steps", 128, 64, 64, 128, 1, 0, 64, "bf16", "lm",
                decode_steps=1024, h0_std=0.1),
    4: Workload(4, "long_mimo_r4_prefill_b1_h64_l32768_q64_then_256_decode", 1, 64, 64, 128, 4, 32768, 64,
                "bf16", "lm", decode_steps=256),
}


def _seed(wid: int, tensor: str, step: int = 0) -> int:
    ss = np.random.SeedSequence([ROOT_SEED, int(wid), _TID[tensor], int(step)])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFF_FFFF_FFFF_FFFF))


def _gen(device, wid, tensor, step=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(wid, tensor, step))
    return g


def _torch_dtype(io_dtype: str) -> torch.dtype:
    if io_dtype == "bf16":
        return torch.bfloat16
    if io_dtype == "f32":
        return torch.float32
    raise ValueError(f"io dtype {io_dtype!r}")


def _normal(shape, g, device, mean=0.0, std=1.0):
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def _uniform(shape, g, device, lo, hi):
    t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def _proj(shape, g, device, dist):
    """B or C: standard normal, then normalised over the last (N) axis."""
    t = _normal(shape, g, device)
    if dist == "tiny":
        t.div_(t.norm(dim=-1, keepdim=True))
    else:
        t.div_(t.pow(2).mean(dim=-1, keepdim=True).sqrt_())
    return t


def _head_params(wid, H, N, dist, device):
    a_hi = math.log(4.0) if dist == "tiny" else math.log(16.0)
    A = -torch.exp(_uniform((H,), _gen(device, wid, "A"), device, math.log(0.5), a_hi))
    omega = _uniform((H, N // 2), _gen(device, wid, "omega"), device, 0.0, math.pi)
    if dist == "tiny":
        D = torch.ones(H, device=device, dtype=torch.float32)
    else:
        D = _normal((H,), _gen(device, wid, "D"), device, 1.0, 0.1)
    return A, omega, D


def _token_tensors(wid, step, b, L, H, G, P, N, R, dist, io_dtype, device):
    dt_ = _torch_dtype(io_dtype)
    x = _normal((b, L, H, R, P), _gen(device, wid, "x", step), device).to(dt_)
    B = _proj((b, L, G, R, N), _gen(device, wid, "B", step), device, dist).to(dt_)
    C = _proj((b, L, G, R, N), _gen(device, wid, "C", step), device, dist).to(dt_)
    dt = torch.nn.functional.softplus(_normal((b, L, H), _gen(device, wid, "dt", step), device, -1.0, 0.5))
    lam = torch.sigmoid(_normal((b, L, H), _gen(device, wid, "lam", step), device))
    return x, B, C, dt.contiguous(), lam.contiguous()


def make_problem(*, batch, seqlen, heads, groups, headdim, dstate, rank, io_dtype="f32",
                 dist="tiny", wid=100, step=0, h0_std=0.0, with_carry=False,
                 device="cpu") -> dict:
    """A prefill problem of any shape with one of the two distribution families.

    `wid` only feeds the seed, so different ids give independent draws.
    """
    if dstate % 2:
        raise ValueError("state dimension N must be even (it is made of rotation pairs)")
    b, L, H, G, P, N, R = batch, seqlen, heads, groups, headdim, dstate, rank
    x, B, C, dt, lam = _token_tensors(wid, step, b, L, H, G, P, N, R, dist, io_dtype, device)
    A, omega, D = _head_params(wid, H, N, dist, device)
    h0 = None
    if h0_std > 0:
        h0 = _normal((b, H, N, P), _gen(device, wid, "h0"), device, 0.0, h0_std)
    carry_B = carry_x = None
    if with_carry:
        dt_ = _torch_dtype(io_dtype)
        carry_B = _proj((b, G, R, N), _gen(device, wid, "carry_B", step), device, dist).to(dt_)
        carry_x = _normal((b, H, R, P), _gen(device, wid, "carry_x", step), device).to(dt_)
    return dict(x=x, dt=dt, A=A, omega=omega, lam=lam, B=B, C=C, D=D, h0=h0,
                carry_B=carry_B, carry_x=carry_x, R=R, io_dtype=io_dtype)


def workload_prefill(wid: int, *, device="cpu", groups=1, seqlen: Optional[int] = None,
                     rank: Optional[int] = None) -> dict:
    """Inputs of a prefill workload (0, 1, 2, or the prefill part of 4)."""
    w = WORKLOADS[wid]
    L = w.seqlen if seqlen is None else seqlen
    R = w.rank if rank is None else rank
    return make_problem(batch=w.batch, seqlen=L, heads=w.heads, groups=groups, headdim=w.headdim,
                        dstate=w.dstate, rank=R, io_dtype=w.io_dtype, dist=w.dist, wid=wid,
                        h0_std=w.h0_std, device=device)


def decode_inputs(wid: int, steps: int, *, device="cpu", groups=1, rank: Optional[int] = None,
                  batch: Optional[int] = None, block: int = 64) -> dict:
    """Per-step inputs of a decode loop, stacked on a leading step axis.

    x: [steps][b][H][R][P], B/C: [steps][b][G][R][N], dt/lam: [steps][b][H].
    Steps are drawn in blocks of `block` steps (block k uses seed step k+1),
    so the first steps do not depend on how many are asked for.
    """
    w = WORKLOADS[wid]
    R = w.rank if rank is None else rank
    b = w.batch if batch is None else batch
    H, P, N, G = w.heads, w.headdim, w.dstate, groups
    xs, Bs, Cs, dts, lams = [], [], [], [], []
    for k in range(0, steps, block):
        n = min(block, steps - k)
        # a block is drawn as a prefill of n tokens, then moved to step-major order
        x, B, C, dt, lam = _token_tensors(wid, 1 + k // block, b, block, H, G, P, N, R, w.dist,
                                          w.io_dtype, device)
        xs.append(x[:, :n].transpose(0, 1))
        Bs.append(B[:, :n].transpose(0, 1))
        Cs.append(C[:, :n].transpose(0, 1))
        dts.append(dt[:, :n].transpose(0, 1))
        lams.append(lam[:, :n].transpose(0, 1))
    A, omega, D = _head_params(wid, H, N, w.dist, device)
    h0 = _normal((b, H, N, P), _gen(device, wid, "h0"), device, 0.0, w.h0_std) if w.h0_std > 0 else None
    cat = lambda ts: torch.cat(ts, 0).contiguous()
    return dict(x=cat(xs), B=cat(Bs), C=cat(Cs), dt=cat(dts), lam=cat(lams), A=A, omega=omega, D=D,
                h0=h0, R=R, io_dtype=w.io_dtype)


def long_sequence(wid: int = 4, *, device="cpu", groups=1, heads: Optional[int] = None) -> dict:
    """Workload 4: one sequence of L + decode_steps tokens, drawn once.

    The first L tokens feed the prefill and the remaining ones the decode steps.
    """
    w = WORKLOADS[wid]
    H = w.heads if heads is None else heads
    return make_problem(batch=w.batch, seqlen=w.seqlen + w.decode_steps, heads=H, groups=groups,
                        headdim=w.headdim, dstate=w.dstate, rank=w.rank, io_dtype=w.io_dtype,
                        dist=w.dist, wid=wid, device=device)


def select_heads(p: dict, heads) -> dict:
    """Sub-problem restricted to the given heads (a gather, no arithmetic).

    B/C are gathered per head (group of head h is h // (H/G)), so the result
    has G' = len(heads) groups unless the problem had G == 1, which is kept.
    """
    heads = list(heads)
    H = p["A"].shape[0]
    G = p["B"].shape[-3]
    idx = torch.tensor(heads, device=p["A"].device)
    out = dict(p)
    out["x"] = p["x"].index_select(-3, idx).contiguous()
    out["dt"] = p["dt"].index_select(-1, idx).contiguous()
    out["lam"] = p["lam"].index_select(-1, idx).contiguous()
    out["A"] = p["A"].index_select(0, idx).contiguous()
    out["D"] = p["D"].index_select(0, idx).contiguous()
    out["omega"] = p["omega"].index_select(0, idx).contiguous()
    if p.get("h0") is not None:
        out["h0"] = p["h0"].index_select(-3, idx).contiguous()
    if p.get("carry_x") is not None:
        out["carry_x"] = p["carry_x"].index_select(-3, idx).contiguous()
    if G != 1:
        gidx = torch.tensor([h // (H // G) for h in heads], device=p["A"].device)
        out["B"] = p["B"].index_select(-3, gidx).contiguous()
        out["C"] = p["C"].index_select(-3, gidx).contiguous()
        if p.get("carry_B") is not None:
            out["carry_B"] = p["carry_B"].index_select(-3, gidx).contiguous()
    return out


def slice_tokens(p: dict, start: int, stop: int) -> dict:
    """Tokens [start, stop) of a prefill problem (no carry or state adjustment)."""
    out = dict(p)
    for k in ("x", "B", "C", "dt", "lam"):
        out[k] = p[k][:, start:stop].contiguous()
    return out


def prologue_inputs(*, tokens, heads, groups, rank, dstate, io_dtype="bf16", wid=200, step=0,
                    device="cpu") -> dict:
    """Raw projections for the input prologue (random draws only, no prologue arithmetic).

    tokens: the token axes, e.g. (b, L) for a prefill or (b,) for a decode step.
    B_raw, C_raw [*tokens][G][R][N] (io dtype): N(0, 1) times a per-row scale
    drawn from U(0.25, 4), so rows arrive at different magnitudes;
    B/C weights ~ N(1, 0.1) and biases ~ N(0, 0.1), [G][R][N] fp32 (stand-ins
    for learned parameters); dt_raw ~ N(-1, 0.5) and lambda_raw ~ N(0, 1)
    [*tokens][H] (softplus and sigmoid of these are the workloads' dt and
    lambda); dt_bias ~ N(0, 0.2) [H].
    """
    tokens = tuple(int(t) for t in tokens)
    G, R, N, H = groups, rank, dstate, heads
    dt_ = _torch_dtype(io_dtype)

    def rows(name):
        t = _normal(tokens + (G, R, N), _gen(device, wid, name, step), device)
        scale = _uniform(tokens + (G, R, 1), _gen(device, wid, "row_scale", step + (0 if name == "B_raw" else 1)),
                         device, 0.25, 4.0)
        return (t * scale).to(dt_)

    par = lambda name, mean, std: _normal((G, R, N), _gen(device, wid, name), device, mean, std)
    return dict(B_raw=rows("B_raw"), C_raw=rows("C_raw"),
                B_weight=par("B_weight", 1.0, 0.1), B_bias=par("B_bias", 0.0, 0.1),
                C_weight=par("C_weight", 1.0, 0.1), C_bias=par("C_bias", 0.0, 0.1),
                dt_raw=_normal(tokens + (H,), _gen(device, wid, "dt_raw", step), device, -1.0, 0.5),
                dt_bias=_normal((H,), _gen(device, wid, "dt_bias"), device, 0.0, 0.2),
                lambda_raw=_normal(tokens + (H,), _gen(device, wid, "lambda_raw", step), device),
                io_dtype=io_dtype)


def mixer_inputs(*, batch, seqlen, d_model, heads, groups, headdim, dstate, rank, wid=500, step=0,
                 device="cpu") -> dict:
    """Synthetic weights and tokens of one mixer block (random draws only).

    u [b][L][d_model] bf16 ~ N(0, 1); projection weights bf16, row-major [out][in]:
    W_x, W_z [H*R*P][d_model] and W_B, W_C [G*R*N][d_model] and W_lambda
    [H][d_model] ~ N(0, 1/d_model) (unit-variance outputs), W_dt [H][d_model] ~
    N(0, 0.25/d_model) with dt_bias [H] ~ N(-1, 0.2) (so dt_raw + bias is near the
    workloads' N(-1, 0.5)), W_out [d_model][H*R*P] ~ N(0, 1/(H*R*P)); B/C weights
    ~ N(1, 0.1), biases ~ N(0, 0.1) [G][R][N] fp32; A, omega, D as the "lm" family.
    Stand-ins for trained weights, which are not available.
    """
    H, G, R, P, N = heads, groups, rank, headdim, dstate
    HRP, GRN = H * R * P, G * R * N
    bf = torch.bfloat16

    def mat(name, rows, cols, std):
        return _normal((rows, cols), _gen(device, wid, name), device, 0.0, std).to(bf)

    A, omega, D = _head_params(wid, H, N, "lm", device)
    par = lambda name, mean, std: _normal((G, R, N), _gen(device, wid, name), device, mean, std)
    return dict(u=_normal((batch, seqlen, d_model), _gen(device, wid, "u", step), device).to(bf),
                W_x=mat("W_x", HRP, d_model, d_model ** -0.5), W_z=mat("W_z", HRP, d_model, d_model ** -0.5),
                W_B=mat("W_B", GRN, d_model, d_model ** -0.5), W_C=mat("W_C", GRN, d_model, d_model ** -0.5),
                W_dt=mat("W_dt", H, d_model, 0.5 * d_model ** -0.5),
                W_lambda=mat("W_lambda", H, d_model, d_model ** -0.5),
                W_out=mat("W_out", d_model, HRP, HRP ** -0.5),
                B_weight=par("B_weight", 1.0, 0.1), B_bias=par("B_bias", 0.0, 0.1),
                C_weight=par("C_weight", 1.0, 0.1), C_bias=par("C_bias", 0.0, 0.1),
                dt_bias=_normal((H,), _gen(device, wid, "dt_bias"), device, -1.0, 0.2),
                A=A, omega=omega, D=D, eps=1e-6, H=H, G=G, R=R, P=P, N=N, d_model=d_model)
