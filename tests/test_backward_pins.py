"""Pins of the oracle's backward pass (oracle/backward.py).

* `backward.forward` (the plain fp64 loop the adjoint differentiates) equals
  the C oracle on the same inputs.
* Every gradient (x, B, C, dt, lambda, A, omega, D, h0, carry_B, carry_x)
  equals a central finite difference of the loss <dy, y> + <dh, h_L> along a
  random direction, with B, C shared by two heads (G = 1) and with one group
  per head. A dropped term, a wrong sign, a transposed product or a missing
  sum over the heads of a group fails the matching case.
* Linearity in x: the x gradient of <dy, y> does not depend on x.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as bw
from mamba_ssm_scan_amd import inputs

NAMES = ["x", "B", "C", "dt", "lam", "A", "omega", "D", "h0", "carry_B", "carry_x"]


def _problem(G, seed):
    p = inputs.make_problem(batch=2, seqlen=9, heads=2, groups=G, headdim=3, dstate=4, rank=2, io_dtype="f32",
                            dist="tiny", wid=700 + seed, h0_std=0.3, with_carry=True)
    return {k: (v.double().numpy() if hasattr(v, "double") else v) for k, v in p.items()}


def _loss(p, dy, dh):
    y, hL = bw.forward(p)
    return float(np.sum(dy * y) + np.sum(dh * hL))


def test_forward_matches_c_oracle():
    p = inputs.make_problem(batch=2, seqlen=17, heads=3, groups=1, headdim=5, dstate=6, rank=3, io_dtype="f32",
                            dist="lm", wid=710, h0_std=0.2, with_carry=True)
    y_c, h_c = oracle.scan(p)
    y, h = bw.forward(p)
    np.testing.assert_allclose(y, y_c, rtol=0, atol=1e-12 * np.abs(y_c).max())
    np.testing.assert_allclose(h, h_c, rtol=0, atol=1e-12 * np.abs(h_c).max())


@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("name", NAMES)
def test_gradient_matches_finite_difference(name, G):
    p = _problem(G, 0)
    rng = np.random.default_rng(11 + G)
    y, hL = bw.forward(p)
    dy = rng.normal(size=y.shape)
    dh = rng.normal(size=hL.shape)
    g = bw.backward(p, dy, dh)[name]
    v = rng.normal(size=np.shape(p[name]))
    eps = 1e-6 * max(1.0, float(np.abs(p[name]).max()))
    pp, pm = dict(p), dict(p)
    pp[name] = p[name] + eps * v
    pm[name] = p[name] - eps * v
    fd = (_loss(pp, dy, dh) - _loss(pm, dy, dh)) / (2 * eps)
    an = float(np.sum(g * v))
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}: finite difference {fd!r}, adjoint {an!r}"


def test_x_gradient_is_independent_of_x():
    p = _problem(1, 1)
    rng = np.random.default_rng(5)
    y, hL = bw.forward(p)
    dy = rng.normal(size=y.shape)
    g1 = bw.backward(p, dy)["x"]
    p2 = dict(p)
    p2["x"] = rng.normal(size=p["x"].shape)
    p2["carry_x"] = p["carry_x"]
    g2 = bw.backward(p2, dy)["x"]
    np.testing.assert_allclose(g1, g2, rtol=1e-12, atol=1e-12)
