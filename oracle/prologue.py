"""Input prologue in fp64 -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may use this
module (see the package header). It shares nothing with the HIP library.

What it computes. The PaperWeekly digest ("复值SSM × 广义梯形离散 × MIMO，线性模型的
全面重构", §2.4 and Fig. 4; §3.4 for the bias's role) places a QK-norm and a
learnable additive bias right after the B/C projection; the workloads draw the
step through softplus and the trapezoid weight through sigmoid. The pages give
no formulas, so the reading taken is:

  B[t,g,r,:] = B_raw[t,g,r,:] / sqrt(mean_n B_raw[t,g,r,n]^2 + eps) * B_weight[g,r,:] + B_bias[g,r,:]
  C[t,g,r,:] likewise with C_weight, C_bias
  dt[t,h]     = softplus(dt_raw[t,h] + dt_bias[h]) = log(1 + e^x)
  lambda[t,h] = sigmoid(lambda_raw[t,h])          = 1 / (1 + e^-x)

(RMS normalisation of each (token, group, rank) row over its N entries, eps
inside the square root, then the elementwise weight, then the bias.) Missing
weights are 1, missing biases 0. Everything in double precision.
"""
from __future__ import annotations

import numpy as np


def softplus(x):
    """log(1 + e^x), through numpy's logaddexp(0, x) (exact for any finite x)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def sigmoid(x):
    """1 / (1 + e^-x); e^-x may overflow to inf for very negative x, giving 0."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def rms_rows(v, eps: float):
    """Each row (last axis) divided by the root of its mean square plus eps."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps)


def qk_norm(raw, weight, bias, eps: float):
    """One of B, C: raw [..., G, R, N]; weight, bias [G, R, N] or None."""
    out = rms_rows(raw, eps)
    if weight is not None:
        out = out * np.asarray(weight, dtype=np.float64)
    if bias is not None:
        out = out + np.asarray(bias, dtype=np.float64)
    return out


def prologue(B_raw=None, C_raw=None, B_weight=None, B_bias=None, C_weight=None, C_bias=None, eps: float = 1e-6,
             dt_raw=None, dt_bias=None, lambda_raw=None):
    """All parts given; returns a dict with B, C, dt, lambda (None where the input was None).

    B_raw, C_raw [..., G, R, N]; dt_raw, lambda_raw [..., H]; dt_bias [H].
    """
    out = {"B": None, "C": None, "dt": None, "lambda": None}
    if B_raw is not None:
        out["B"] = qk_norm(B_raw, B_weight, B_bias, eps)
    if C_raw is not None:
        out["C"] = qk_norm(C_raw, C_weight, C_bias, eps)
    if dt_raw is not None:
        x = np.asarray(dt_raw, dtype=np.float64)
        if dt_bias is not None:
            x = x + np.asarray(dt_bias, dtype=np.float64)
        out["dt"] = softplus(x)
    if lambda_raw is not None:
        out["lambda"] = sigmoid(lambda_raw)
    return out
