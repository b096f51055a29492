"""Pins of the oracle's input prologue (oracle/prologue.py) against mathematics.

The pages name the parts (a QK-norm and a learnable bias after the B/C
projection: "复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构", §2.4; softplus and
sigmoid in the workloads' input recipe) but print no formula or worked value.
Each pin below checks a property that a plausible slip breaks:

  softplus: value ln 2 at 0, the identity softplus(x) - softplus(-x) = x
            (breaks for log(1 + e^-x), a missing log, a sign slip), linear
            growth for large x, and its derivative equals sigmoid.
  sigmoid:  1/2 at 0, sigmoid(x) + sigmoid(-x) = 1, the logistic closed form
            at x = ln 3 (= 3/4).
  QK-norm:  unit mean square per row (weight 1, bias 0, eps 0), invariance to
            a positive row scale, oddness, a two-entry row by hand, the order
            normalise -> weight -> bias, eps keeping a zero row finite, and the
            row axis being N (not R or G).
  dt bias:  added before softplus.
"""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_softplus_values_and_identities():
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=0, abs=1e-16)
    rng = np.random.default_rng(7)
    x = rng.normal(0, 5, size=1000)
    np.testing.assert_allclose(oracle.softplus(x) - oracle.softplus(-x), x, rtol=0, atol=1e-12)
    big = np.array([40.0, 100.0, 700.0])
    np.testing.assert_allclose(oracle.softplus(big), big, rtol=1e-15)
    assert oracle.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)
    assert np.all(oracle.softplus(x) > 0)


def test_softplus_derivative_is_sigmoid():
    x = np.linspace(-8, 8, 161)
    h = 1e-5
    d = (oracle.softplus(x + h) - oracle.softplus(x - h)) / (2 * h)
    np.testing.assert_allclose(d, oracle.sigmoid(x), rtol=0, atol=1e-9)


def test_sigmoid_values_and_symmetry():
    assert oracle.sigmoid(0.0) == 0.5
    assert oracle.sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    x = np.random.default_rng(8).normal(0, 6, size=1000)
    np.testing.assert_allclose(oracle.sigmoid(x) + oracle.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert oracle.sigmoid(-1000.0) == 0.0 and oracle.sigmoid(1000.0) == 1.0


def test_qk_norm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(9)
    raw = rng.normal(0, 3, size=(5, 2, 3, 16))
    out = oracle.qk_norm(raw, None, None, 0.0)
    np.testing.assert_allclose(np.mean(out ** 2, axis=-1), 1.0, rtol=0, atol=1e-14)
    alpha = rng.uniform(0.1, 10, size=(5, 2, 3, 1))
    np.testing.assert_allclose(oracle.qk_norm(raw * alpha, None, None, 0.0), out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.qk_norm(-raw, None, None, 0.0), -out, rtol=0, atol=0)


def test_qk_norm_two_entry_row_by_hand():
    # row (3, 4): mean square (9 + 16) / 2 = 12.5
    out = oracle.qk_norm(np.array([[[[3.0, 4.0]]]]), None, None, 0.0)
    np.testing.assert_allclose(out[0, 0, 0], [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    # with eps: the square root holds mean square + eps
    out = oracle.qk_norm(np.array([[[[3.0, 4.0]]]]), None, None, 0.5)
    np.testing.assert_allclose(out[0, 0, 0], [3 / math.sqrt(13.0), 4 / math.sqrt(13.0)], rtol=1e-15)


def test_qk_norm_order_weight_then_bias():
    rng = np.random.default_rng(10)
    G, R, N = 2, 3, 8
    raw = rng.normal(size=(4, G, R, N))
    w = rng.uniform(0.5, 2.0, size=(G, R, N))
    bias = rng.normal(size=(G, R, N))
    out = oracle.qk_norm(raw, w, bias, 0.0)
    # undo bias then weight: the rows have unit mean square again
    np.testing.assert_allclose(np.mean(((out - bias) / w) ** 2, axis=-1), 1.0, rtol=0, atol=1e-13)
    # the bias is not normalised away: a constant raw row leaves w + bias (up to sign)
    const = np.ones((1, G, R, N)) * 2.5
    np.testing.assert_allclose(oracle.qk_norm(const, w, bias, 0.0)[0], w + bias, rtol=1e-15)


def test_qk_norm_eps_keeps_zero_rows_finite():
    bias = np.arange(1 * 1 * 4, dtype=np.float64).reshape(1, 1, 4)
    out = oracle.qk_norm(np.zeros((3, 1, 1, 4)), None, bias, 1e-6)
    np.testing.assert_array_equal(out, np.broadcast_to(bias, (3, 1, 1, 4)))


def test_qk_norm_row_axis_is_the_state_axis():
    # one (token, group, rank) row scaled by 10 changes no other row
    rng = np.random.default_rng(11)
    raw = rng.normal(size=(3, 2, 2, 8))
    scaled = raw.copy()
    scaled[1, 0, 1] *= 10.0
    np.testing.assert_allclose(oracle.qk_norm(scaled, None, None, 0.0), oracle.qk_norm(raw, None, None, 0.0),
                               rtol=0, atol=1e-14)


def test_prologue_dt_bias_enters_before_softplus():
    rng = np.random.default_rng(12)
    raw = rng.normal(-1, 0.5, size=(2, 6, 4))
    bias = rng.normal(size=4)
    got = oracle.prologue(dt_raw=raw, dt_bias=bias)["dt"]
    np.testing.assert_allclose(got, oracle.prologue(dt_raw=raw + bias)["dt"], rtol=1e-15)
    lam = oracle.prologue(lambda_raw=raw)["lambda"]
    np.testing.assert_allclose(lam, 1 - oracle.prologue(lambda_raw=-raw)["lambda"], rtol=0, atol=1e-15)
    assert oracle.prologue(B_raw=None)["B"] is None
