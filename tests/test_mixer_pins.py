"""Pins of the mixer-block oracle (oracle/mixer.py), each an independent route.

* silu by values and identities: silu(0) = 0, silu(ln 3) = (3/4) ln 3 (sigmoid(ln 3)
  = 3/4), silu(v) - silu(-v) = v, silu(v) -> v for large v.
* bf16 rounding: representable values pass unchanged; halfway cases go to the
  even neighbour; a value just above halfway rounds up.
* A zero z projection closes the gate: the output is exactly zero.
* A zero B projection (no B bias) removes the recurrence's input, leaving the
  skip path: out = ((D x) * silu(z)) W_out written out by hand.
* One token from a zero state: y_r = gamma sum_r' (C_r . B_r') x_r' + D x_r, a
  closed form of the whole block (with the prologue's own pinned formulas).
* Causality and batch independence: perturbing token t0 leaves earlier outputs
  bit-identical; permuting the batch permutes the output.
* The block over L tokens equals the block over the first k tokens followed by
  the rest started from the state h_k and the carry of token k - 1 (written
  out with the recurrence oracle), so prefill-then-decode is the same function.
Run with io_round=False (fp64 throughout) except for the rounding pins.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import mixer
from mamba_ssm_scan_amd import inputs


def _w(**kw):
    args = dict(batch=2, seqlen=6, d_model=24, heads=2, groups=1, headdim=4, dstate=6, rank=2)
    args.update(kw)
    return inputs.mixer_inputs(**args)


def _np(t):
    return t.double().numpy() if hasattr(t, "double") else np.asarray(t, dtype=np.float64)


def test_silu_values():
    assert mixer.silu(0.0) == 0.0
    assert math.isclose(float(mixer.silu(math.log(3.0))), 0.75 * math.log(3.0), rel_tol=1e-15)
    v = np.linspace(-6, 6, 49)
    np.testing.assert_allclose(mixer.silu(v) - mixer.silu(-v), v, rtol=0, atol=1e-14)
    assert math.isclose(float(mixer.silu(40.0)), 40.0, rel_tol=1e-15)
    assert abs(float(mixer.silu(-40.0))) < 1e-15


def test_round_bf16():
    exact = np.array([0.0, 1.0, -2.5, 0.15625, 3.0 * 2 ** -130, 65280.0])
    np.testing.assert_array_equal(mixer.round_bf16(exact), exact)
    ulp = 2.0 ** -7  # bf16 spacing at 1
    assert mixer.round_bf16(1.0 + ulp / 2) == 1.0                     # tie -> even (1.0)
    assert mixer.round_bf16(1.0 + 3 * ulp / 2) == 1.0 + 2 * ulp       # tie -> even (1 + 2 ulp)
    assert mixer.round_bf16(1.0 + ulp / 2 + 2 ** -20) == 1.0 + ulp    # above the tie
    assert mixer.round_bf16(-(1.0 + ulp / 2 + 2 ** -20)) == -(1.0 + ulp)


def test_zero_gate_gives_zero():
    w = _w()
    w["W_z"] = w["W_z"] * 0
    out, _, _ = mixer.forward(w, w["u"], io_round=False)
    assert np.all(out == 0.0)


def test_skip_path_alone():
    """B projection and bias zero: U = 0, so y = D x and the block is a closed form."""
    w = _w()
    w["W_B"] = w["W_B"] * 0
    w["B_bias"] = None
    out, _, _ = mixer.forward(w, w["u"], io_round=False)
    u = _np(w["u"])
    b, L, _ = u.shape
    H, R, P = w["H"], w["R"], w["P"]
    x = (u @ _np(w["W_x"]).T).reshape(b, L, H, R, P)
    z = (u @ _np(w["W_z"]).T).reshape(b, L, H, R, P)
    y = _np(w["D"])[None, None, :, None, None] * x
    ref = (y * z / (1.0 + np.exp(-z))).reshape(b, L, -1) @ _np(w["W_out"]).T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_single_token_closed_form():
    w = _w(seqlen=1, groups=2, rank=3)
    out, hL, parts = mixer.forward(w, w["u"], io_round=False)
    u = _np(w["u"])
    b = u.shape[0]
    H, G, R, P, N = w["H"], w["G"], w["R"], w["P"], w["N"]
    x = (u @ _np(w["W_x"]).T).reshape(b, H, R, P)
    z = (u @ _np(w["W_z"]).T).reshape(b, H, R, P)

    def qk(raw, wt, bias):
        r = raw / np.sqrt(np.mean(raw * raw, axis=-1, keepdims=True) + w["eps"])
        return r * _np(wt) + _np(bias)

    Bm = qk((u @ _np(w["W_B"]).T).reshape(b, G, R, N), w["B_weight"], w["B_bias"])
    Cm = qk((u @ _np(w["W_C"]).T).reshape(b, G, R, N), w["C_weight"], w["C_bias"])
    dt = np.log1p(np.exp((u @ _np(w["W_dt"]).T).reshape(b, H) + _np(w["dt_bias"])))
    lam = 1.0 / (1.0 + np.exp(-(u @ _np(w["W_lambda"]).T).reshape(b, H)))
    y = np.empty((b, H, R, P))
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            gram = Cm[bb, g] @ Bm[bb, g].T            # [R][R']: C_r . B_r'
            y[bb, h] = lam[bb, h] * dt[bb, h] * (gram @ x[bb, h]) + _np(w["D"])[h] * x[bb, h]
    ref = (y * z / (1.0 + np.exp(-z))).reshape(b, 1, -1) @ _np(w["W_out"]).T
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_causal_and_batch_independent():
    w = _w(seqlen=7)
    out, _, _ = mixer.forward(w, w["u"], io_round=False)
    u2 = w["u"].clone()
    u2[:, 4] += 1.0
    out2, _, _ = mixer.forward(w, u2, io_round=False)
    np.testing.assert_array_equal(out[:, :4], out2[:, :4])
    assert np.abs(out[:, 4:] - out2[:, 4:]).max() > 1e-3
    out3, _, _ = mixer.forward(w, w["u"].flip(0), io_round=False)
    np.testing.assert_allclose(out3, out[::-1], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("k", [1, 4])
def test_split_equals_whole(k):
    """Tokens [0, L) at once = tokens [0, k), then [k, L) from (h_k, carry of token k-1)."""
    w = _w(seqlen=7)
    out, hL, parts = mixer.forward(w, w["u"], io_round=False)
    _, hk, pk = mixer.forward(w, w["u"][:, :k], io_round=False)
    _, _, pr = mixer.forward(w, w["u"][:, k:], io_round=False)
    from oracle.backward import forward as fwd64
    q = {"x": pr["x"], "dt": pr["dt"], "lam": pr["lam"], "B": pr["B"], "C": pr["C"], "A": _np(w["A"]),
         "omega": _np(w["omega"]), "D": _np(w["D"]), "h0": hk, "carry_B": pk["B"][:, k - 1],
         "carry_x": pk["x"][:, k - 1]}
    y_rest, h_rest = fwd64(q)
    np.testing.assert_allclose(y_rest, parts["y"][:, k:], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(h_rest, hL, rtol=1e-11, atol=1e-12)
