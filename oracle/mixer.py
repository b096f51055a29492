"""The mixer block around the recurrence, in fp64 -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may use this
module (see the package header). It shares nothing with the HIP library.

What it computes. The PaperWeekly digest ("复值SSM × 广义梯形离散 × MIMO，线性模型的
全面重构", §2.4 and Fig. 4) lists what one Mamba-3 SSM block holds: the complex
(rotating) state with the trapezoid rule, MIMO inputs, QK-norm plus a learnable
bias after the B/C projection, and no short convolution. It prints no block
formula; the reading taken is the Mamba-2 block the pages compare against, with
those changes: per token u_t (d_model entries)

  x      = u W_x^T      z = u W_z^T           [H][R][P] each (one row block of W per head and rank)
  B_raw  = u W_B^T      C_raw = u W_C^T       [G][R][N]
  dt_raw = u W_dt^T     lambda_raw = u W_lambda^T   [H]
  B, C, dt, lambda = prologue(B_raw, C_raw, dt_raw, lambda_raw)   (QK-norm + bias, softplus, sigmoid)
  y      = the recurrence over the tokens (x, dt, A, omega, lambda, B, C, D)
  out    = (y * silu(z)) W_out^T                silu(v) = v * sigmoid(v)

Weights are row-major [out][in], as a linear layer stores them. With io_round
(the default) the values the block hands between its stages in bf16 -- x, z, B_raw, C_raw, B, C, y and the
gated y -- are rounded to bf16 (nearest, ties to even) where they are formed,
as the block's storage types say; dt_raw, lambda_raw, dt and lambda stay fp32
(dt, lambda rounded to fp32). Everything else is double precision. With
io_round=False the same steps run in fp64 throughout (the mathematical block).
"""
from __future__ import annotations

import numpy as np

from . import scan
from .prologue import prologue, sigmoid


def _np64(a):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


def round_bf16(a):
    """Nearest bf16 value (ties to even) of each entry, returned as float64.

    Through float32 (the kernels round fp32 values); NaN and infinities pass.
    """
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    finite = np.isfinite(f)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = np.where(finite, rounded, u).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


def silu(v):
    """v * sigmoid(v)."""
    v = np.asarray(v, dtype=np.float64)
    return v * sigmoid(v)


def forward(w: dict, u, h0=None, io_round: bool = True, nthreads=None):
    """Block output for tokens u [b][L][d_model]; returns (out [b][L][d_model], h_L, parts).

    w: W_x, W_z [H*R*P][d_model]; W_B, W_C [G*R*N][d_model]; W_dt, W_lambda
    [H][d_model]; W_out [d_model][H*R*P]; B_weight, B_bias, C_weight, C_bias
    [G][R][N] (or None); dt_bias [H] (or None); A, D [H]; omega [H][N/2]; eps;
    and the sizes H, G, R, P, N. parts holds the intermediate tensors.
    """
    rb = round_bf16 if io_round else (lambda a: np.asarray(a, dtype=np.float64))
    f32 = (lambda a: np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)) if io_round else rb
    H, G, R, P, N = (int(w[k]) for k in ("H", "G", "R", "P", "N"))
    u = _np64(u)
    b, L, dm = u.shape
    W = {k: _np64(w[k]).T for k in ("W_x", "W_z", "W_B", "W_C", "W_dt", "W_lambda", "W_out")}  # [in][out] views
    x = rb(u @ W["W_x"]).reshape(b, L, H, R, P)
    z = rb(u @ W["W_z"]).reshape(b, L, H, R, P)
    B_raw = rb(u @ W["W_B"]).reshape(b, L, G, R, N)
    C_raw = rb(u @ W["W_C"]).reshape(b, L, G, R, N)
    dt_raw = f32(u @ W["W_dt"])
    lam_raw = f32(u @ W["W_lambda"])
    pro = prologue(B_raw=B_raw, C_raw=C_raw, B_weight=_np64(w.get("B_weight")), B_bias=_np64(w.get("B_bias")),
                   C_weight=_np64(w.get("C_weight")), C_bias=_np64(w.get("C_bias")), eps=float(w["eps"]),
                   dt_raw=dt_raw, dt_bias=_np64(w.get("dt_bias")), lambda_raw=lam_raw)
    Bn, Cn = rb(pro["B"]), rb(pro["C"])
    dt, lam = f32(pro["dt"]), f32(pro["lambda"])
    p = {"x": x, "dt": dt, "lam": lam, "B": Bn, "C": Cn, "A": _np64(w["A"]), "omega": _np64(w["omega"]),
         "D": _np64(w["D"]), "h0": _np64(h0)}
    if io_round:
        y, hL = scan(p, nthreads=nthreads)
    else:
        y, hL = _scan64(p)
    y = rb(y)
    g = rb(y * silu(z))
    out = g.reshape(b, L, H * R * P) @ W["W_out"]
    parts = {"x": x, "z": z, "B": Bn, "C": Cn, "dt": dt, "lam": lam, "y": y, "gated": g}
    return out, hL, parts


def _scan64(p):
    """The recurrence in fp64 on fp64 inputs (the C oracle takes fp32 carriers)."""
    from .backward import forward as fwd64
    return fwd64({k: v for k, v in p.items()})
