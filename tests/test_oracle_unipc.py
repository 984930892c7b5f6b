"""Pins of the oracle's UniPC solver (published method restated; the pages print no formula).

* Order 1 is the Euler step of the flow ODE, including steps from t = 0 and to t = 1 (closed form:
  both are x + (t - s) v).
* A UniPC update integrates the data-prediction ODE exactly when the data prediction is a
  polynomial in lambda = log(t / (1 - t)) of degree below the predictor's order (degree up to the
  order for the corrector): the exact solution is (sigma_t/sigma_s) x_s + sigma_t * integral of
  e^lambda x_hat(lambda) between the two half log-SNRs, written out here with the antiderivatives
  of lambda^k e^lambda. One degree more is not integrated exactly (the pin has teeth).
* The whole loop on a straight-line flow (constant velocity) ends at x_0 + v for every order.
* The loop with the predictor alone at order 1 equals the oracle's Euler loop.
"""
import math

import numpy as np
import pytest

import oracle as O

lam = lambda t: math.log(t / (1.0 - t))  # noqa: E731


def _antider(l, c):
    # integral of e^l (c0 + c1 l + c2 l^2 + c3 l^3) dl
    return math.exp(l) * (c[0] + c[1] * (l - 1) + c[2] * (l * l - 2 * l + 2) + c[3] * (l ** 3 - 3 * l * l + 6 * l - 6))


def _exact(xs, ts, tt, c):
    return (1 - tt) / (1 - ts) * xs + (1 - tt) * (_antider(lam(tt), c) - _antider(lam(ts), c))


def _xhat(c):
    return lambda t: sum(ck * lam(t) ** k for k, ck in enumerate(c))


@pytest.mark.parametrize("order", [1, 2, 3])
def test_polynomial_data_prediction_is_integrated_exactly(order):
    hist = [0.52, 0.43, 0.31]
    ts, tt, xs = hist[0], 0.64, 1.3
    rng = np.random.default_rng(order)
    for deg in range(4):
        c = list(rng.standard_normal(deg + 1)) + [0.0] * (3 - deg)
        xh = _xhat(c)
        a, w = O.update_weights(tt, hist[:order], corrector=False)
        pred = a * xs + sum(wi * xh(ti) for wi, ti in zip(w, hist[:order]))
        a, wc = O.update_weights(tt, hist[:order], corrector=True)
        corr = a * xs + sum(wi * xh(ti) for wi, ti in zip(wc, hist[:order])) + wc[-1] * xh(tt)
        ref = _exact(xs, ts, tt, c)
        scale = 1.0 + abs(ref)
        if deg < order:
            assert abs(pred - ref) <= 1e-12 * scale
        elif deg == order:
            assert abs(pred - ref) > 1e-6 * scale
        if deg <= order:
            assert abs(corr - ref) <= 1e-12 * scale
        else:
            assert abs(corr - ref) > 1e-6 * scale


@pytest.mark.parametrize("ts,tt", [(0.0, 1 / 16), (0.3, 0.45), (15 / 16, 1.0), (0.0, 1.0)])
def test_order_one_is_the_euler_step(ts, tt):
    x, v = 0.8, -1.3
    a, w = O.update_weights(tt, [ts], corrector=False)
    assert abs(a * x + w[0] * (x + (1 - ts) * v) - (x + (tt - ts) * v)) <= 1e-15


def test_step_orders_on_the_uniform_grid():
    grid = [k / 16 for k in range(17)]
    orders = [O.step_order(grid, k, 2) for k in range(16)]
    assert orders[0] == 1 and orders[1] == 1 and orders[-1] == 1      # lambda infinite at t = 0 and t = 1
    assert all(o == 2 for o in orders[2:-1])
    assert [O.step_order(grid, k, 3) for k in range(2, 5)] == [2, 3, 3]


@pytest.mark.parametrize("order", [1, 2, 3])
def test_straight_line_flow_is_exact(order):
    rng = np.random.default_rng(5)
    x0v, x0a = rng.standard_normal((6, 4)), rng.standard_normal((3, 2))
    vv, va = rng.standard_normal((6, 4)), rng.standard_normal((3, 2))
    grid = [k / 16 for k in range(17)]
    xv, xa, calls, flags = O.denoise_chunk_unipc(lambda a, b, t: (vv, va), x0v, x0a, grid, 2.0, order=order)
    assert calls == 16 and not any(flags)
    np.testing.assert_allclose(xv, x0v + vv, atol=1e-12)
    np.testing.assert_allclose(xa, x0a + va, atol=1e-12)


def test_order_one_loop_equals_euler_loop():
    rng = np.random.default_rng(6)
    x0v, x0a = rng.standard_normal((5, 3)), rng.standard_normal((2, 2))
    A, B = rng.standard_normal((3, 3)) * 0.3, rng.standard_normal((2, 2)) * 0.3

    def dit(xv, xa, t):   # a smooth nonlinear velocity field
        return np.tanh(xv @ A) * (1 + t), np.sin(xa @ B) - t

    grid = [k / 16 for k in range(17)]
    u = O.denoise_chunk_unipc(dit, x0v, x0a, grid, 2.0, order=1, corrector=False)
    e = O.denoise_chunk(dit, x0v, x0a, grid, 2.0)
    np.testing.assert_allclose(u[0], e[0], atol=1e-12)
    np.testing.assert_allclose(u[1], e[1], atol=1e-12)
    # the corrector, and a higher order, change the result on a curved field
    for kw in (dict(order=1), dict(order=2, corrector=False), dict(order=2)):
        h = O.denoise_chunk_unipc(dit, x0v, x0a, grid, 2.0, **kw)
        assert np.abs(h[0] - e[0]).max() > 1e-6
