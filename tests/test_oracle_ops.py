"""Pins of the oracle's elementary operations against library routines, closed forms and brute force.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign or index,
a transposed operand) fails it; none re-types the oracle's own formula.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

RNG = np.random.default_rng(1140)


def _r(*shape, dt=np.float32):
    return RNG.standard_normal(shape).astype(dt)


def test_layer_norm_matches_torch():
    x = _r(7, 300) * 3 + 1.5
    w, b = _r(300), _r(300)
    ref = F.layer_norm(torch.from_numpy(x), (300,), torch.from_numpy(w), torch.from_numpy(b), eps=1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(x, 1e-6, w, b), ref, rtol=0, atol=2e-6)
    ref0 = F.layer_norm(torch.from_numpy(x), (300,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.layer_norm(x, 1e-6), ref0, rtol=0, atol=2e-6)


def test_rms_norm_matches_torch():
    x = _r(5, 512) * 0.3
    g = _r(512)
    ref = F.rms_norm(torch.from_numpy(x), (512,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, 1e-6, g), ref, rtol=1e-6, atol=1e-6)


def test_gelu_tanh_and_silu_match_torch():
    x = np.linspace(-8, 8, 4001, dtype=np.float32)
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(O.gelu_tanh(x), ref, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(O.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-6, atol=1e-6)


def test_modulated_norm_statistics():
    # After adaLN with a per-row constant shift s and scale c, every row has mean s and std (1 + c):
    # pins both the (1 + scale) form and which vector is the shift.
    x = _r(6, 1024, dt=np.float64) * 4 - 2
    shift = np.full((6, 1), 0.7)
    scale = np.linspace(-0.5, 2.0, 6)[:, None]
    y = O.modulated_norm(x, shift, scale, 1e-12)
    np.testing.assert_allclose(y.mean(axis=1), 0.7, atol=1e-12)
    np.testing.assert_allclose(y.std(axis=1), 1.0 + scale[:, 0], rtol=1e-9)


def test_modulated_rms_norm_matches_torch():
    # The RMSNorm variant of the block norms: torch's rms_norm, then the same (1 + scale), shift; the
    # result differs from the LayerNorm form exactly when the rows have a non-zero mean.
    x = _r(5, 768, dt=np.float64) * 4 - 1.5
    shift = _r(1, 768, dt=np.float64) - 0.5
    scale = _r(1, 768, dt=np.float64) - 0.5
    ref = F.rms_norm(torch.from_numpy(x), (768,), eps=1e-6).numpy() * (1 + scale) + shift
    np.testing.assert_allclose(O.modulated_norm(x, shift, scale, 1e-6, rms=True), ref, rtol=1e-12, atol=1e-12)
    xc = x - x.mean(axis=1, keepdims=True)
    np.testing.assert_allclose(O.modulated_norm(xc, shift, scale, 1e-6, rms=True),
                               O.modulated_norm(xc, shift, scale, 1e-6), rtol=1e-9, atol=1e-9)
    assert np.abs(O.modulated_norm(x, shift, scale, 1e-6, rms=True) - O.modulated_norm(x, shift, scale, 1e-6)).max() > 0.1


def test_linear_brute_force():
    x, w, b = _r(3, 5, dt=np.float64), _r(4, 5, dt=np.float64), _r(4, dt=np.float64)
    y = O.linear(x, w, b)
    for i, j in itertools.product(range(3), range(4)):
        assert abs(y[i, j] - (sum(x[i, k] * w[j, k] for k in range(5)) + b[j])) < 1e-12


def _attention_loops(q, k, v, visible):
    H, Lq, d = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(Lq):
            js = [j for j in range(k.shape[1]) if visible is None or visible[i, j]]
            s = [sum(q[h, i, c] * k[h, j, c] for c in range(d)) / math.sqrt(d) for j in js]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for c in range(d):
                out[h, i, c] = sum(e[n] * v[h, j, c] for n, j in enumerate(js)) / z
    return out


@pytest.mark.parametrize("Lq,Lk,masked", [(1, 1, False), (5, 9, False), (8, 16, True), (3, 7, True)])
def test_attention_brute_force(Lq, Lk, masked):
    H, d = 2, 4
    q, k, v = _r(H, Lq, d, dt=np.float64), _r(H, Lk, d, dt=np.float64), _r(H, Lk, d, dt=np.float64)
    vis = None
    if masked:
        vis = RNG.random((Lq, Lk)) < 0.6
        vis[:, 0] = True
    np.testing.assert_allclose(O.attention(q, k, v, vis), _attention_loops(q, k, v, vis), rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa_with_mask():
    H, Lq, Lk, d = 3, 12, 20, 16
    q, k, v = _r(H, Lq, d), _r(H, Lk, d), _r(H, Lk, d)
    vis = RNG.random((Lq, Lk)) < 0.5
    vis[:, 3] = True
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=torch.from_numpy(vis)).numpy()
    np.testing.assert_allclose(O.attention(q, k, v, vis), ref, rtol=1e-5, atol=1e-6)


def test_attention_special_cases():
    H, d = 2, 8
    v1 = _r(H, 1, d)
    assert np.array_equal(O.attention(_r(H, 4, d), _r(H, 1, d), v1, None), np.repeat(v1, 4, axis=1))
    v = _r(H, 10, d, dt=np.float64)
    o = O.attention(np.zeros((H, 3, d)), _r(H, 10, d, dt=np.float64), v, None)
    np.testing.assert_allclose(o, np.repeat(v.mean(axis=1, keepdims=True), 3, axis=1), atol=1e-14)


def test_attention_hidden_keys_cannot_leak():
    H, Lq, Lk, d = 1, 4, 6, 8
    q, k, v = _r(H, Lq, d), _r(H, Lk, d), _r(H, Lk, d)
    vis = np.ones((Lq, Lk), bool)
    vis[:, 4:] = False
    k2, v2 = k.copy(), v.copy()
    k2[:, 4:] = 1e30
    v2[:, 4:] = -3e30
    assert np.array_equal(O.attention(q, k, v, vis), O.attention(q, k2, v2, vis))


def test_sinusoid_closed_forms():
    # t = 1 (clean) -> s = 0 -> cos half all ones, sin half all zeros, exactly.
    e = O.timestep_sinusoid(1.0, 256)
    assert np.array_equal(e, np.concatenate([np.ones(128), np.zeros(128)]).astype(np.float32))
    # w_64 = 10000^(-1/2) = 1/100 and w_0 = 1: with s = 100*pi, entry 64 is cos(pi) = -1 and
    # entry 0 is cos(100*pi) = 1; the sin half at 64 is sin(pi) = 0.
    e = O.timestep_sinusoid(1.0 - 0.1 * math.pi, 256, dt=np.float64)
    assert abs(e[64] + 1.0) < 1e-12 and abs(e[0] - 1.0) < 1e-9 and abs(e[128 + 64]) < 1e-12


def test_rope_split_and_frequencies():
    assert O.rope_axis_split(128) == (44, 42, 42)
    assert O.rope_axis_split(64) == (24, 20, 20)
    axis, freq = O.rope_frequencies(128, 10000.0)
    assert list(np.bincount(axis)) == [22, 21, 21]
    # the first pair of every axis turns by exactly its position (frequency 1)
    assert freq[0] == 1.0 and freq[22] == 1.0 and freq[43] == 1.0


def test_rope_d2_is_plain_rotation_and_preserves_norm():
    # head_dim 2 -> a single frame-axis pair with frequency 1: the textbook 2-D rotation by the frame.
    x = _r(5, 1, 2, dt=np.float64)
    pos = np.array([[f, 0, 0] for f in range(5)])
    y = O.apply_rope(x, pos, 2, 10000.0)
    for f in range(5):
        c, s = math.cos(f), math.sin(f)
        np.testing.assert_allclose(y[f, 0], [c * x[f, 0, 0] - s * x[f, 0, 1], s * x[f, 0, 0] + c * x[f, 0, 1]], atol=1e-14)
    x = _r(9, 3, 128, dt=np.float64)
    pos = RNG.integers(0, 50, size=(9, 3))
    y = O.apply_rope(x, pos, 128, 10000.0)
    n = lambda a: a[..., 0::2] ** 2 + a[..., 1::2] ** 2  # noqa: E731
    np.testing.assert_allclose(n(y), n(x), rtol=1e-12)


def test_rope_relative_positions():
    # <R(p) q, R(p') k> depends only on p - p': shift both by the same offset on every axis.
    q, k = _r(1, 2, 64, dt=np.float64), _r(1, 2, 64, dt=np.float64)
    p, pk = np.array([[3, 4, 5]]), np.array([[1, 7, 2]])
    for delta in ([10, 0, 0], [0, 3, 0], [2, 5, 11]):
        d = np.array([delta])
        a = np.sum(O.apply_rope(q, p, 64, 1e4) * O.apply_rope(k, pk, 64, 1e4), axis=-1)
        b = np.sum(O.apply_rope(q, p + d, 64, 1e4) * O.apply_rope(k, pk + d, 64, 1e4), axis=-1)
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_cfg_special_cases():
    v = _r(2, 50, 8)
    assert np.array_equal(O.cfg_combine(v, 1.0), v[0])
    assert np.array_equal(O.cfg_combine(v, 0.0), v[1])


@pytest.mark.parametrize("t", [0.0, 0.25, 0.5, 0.9375, 1.0])
def test_one_euler_step_recovers_clean_data(t):
    # x_t + (1 - t)(x1 - eps) = x1: exact algebra, rounding within a few ulp of max(|x1|, |eps|).
    x1, eps = _r(4096), _r(4096)
    xt = O.interpolate(x1, eps, t)
    x = O.euler_update(xt, x1 - eps, t, 1.0)
    tol = 4 * np.spacing(np.maximum(np.abs(x1), np.abs(eps)).astype(np.float32))
    assert np.all(np.abs(x - x1) <= tol)
    if t == 1.0:
        assert np.array_equal(x, x1)


def test_cosine_fp64():
    a = _r(1000)
    assert abs(O.cosine_fp64(a, a) - 1.0) < 1e-14
    assert abs(O.cosine_fp64(a, -a) + 1.0) < 1e-14
    assert abs(O.cosine_fp64(np.array([1.0, 0.0]), np.array([0.0, 2.0]))) == 0.0


def test_swiglu_feed_forward_structure():
    # SwiGLU variant: the up rows (odd rows of W1) enter linearly, the gate rows through SiLU. Scaling
    # the up rows and biases by a scales the product by a; a zero gate leaves only b2; an up path
    # fixed at 1 leaves a SiLU feed-forward, checked against torch.
    from types import SimpleNamespace
    rng = np.random.default_rng(11)
    D, Fh = 32, 24
    w = SimpleNamespace(variant=4)
    lp = {"w_ff1": rng.standard_normal((2 * Fh, D)) * 0.3, "b_ff1": rng.standard_normal(2 * Fh) * 0.1,
          "w_ff2": rng.standard_normal((D, Fh)) * 0.3, "b_ff2": rng.standard_normal(D) * 0.1}
    y = rng.standard_normal((7, D))
    base = O.feed_forward(w, lp, y)
    lp2 = dict(lp, w_ff1=lp["w_ff1"].copy(), b_ff1=lp["b_ff1"].copy())
    lp2["w_ff1"][1::2] *= 2.5
    lp2["b_ff1"][1::2] *= 2.5
    np.testing.assert_allclose(O.feed_forward(w, lp2, y) - lp["b_ff2"], 2.5 * (base - lp["b_ff2"]), rtol=1e-12, atol=1e-12)
    lp3 = dict(lp, w_ff1=lp["w_ff1"].copy(), b_ff1=lp["b_ff1"].copy())
    lp3["w_ff1"][0::2] = 0.0
    lp3["b_ff1"][0::2] = 0.0
    np.testing.assert_array_equal(O.feed_forward(w, lp3, y), np.broadcast_to(lp["b_ff2"], (7, D)))
    lp4 = dict(lp, w_ff1=lp["w_ff1"].copy(), b_ff1=lp["b_ff1"].copy())
    lp4["w_ff1"][1::2] = 0.0
    lp4["b_ff1"][1::2] = 1.0
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    ref = F.linear(F.silu(F.linear(t(y), t(lp["w_ff1"][0::2]), t(lp["b_ff1"][0::2]))), t(lp["w_ff2"]), t(lp["b_ff2"]))
    np.testing.assert_allclose(O.feed_forward(w, lp4, y), ref.numpy(), rtol=1e-12, atol=1e-12)
    # the adopted GELU-tanh feed-forward against torch
    w0 = SimpleNamespace(variant=0)
    lp0 = dict(lp, w_ff1=lp["w_ff1"][:Fh], b_ff1=lp["b_ff1"][:Fh])
    ref0 = F.linear(F.gelu(F.linear(t(y), t(lp0["w_ff1"]), t(lp0["b_ff1"])), approximate="tanh"), t(lp["w_ff2"]),
                    t(lp["b_ff2"]))
    np.testing.assert_allclose(O.feed_forward(w0, lp0, y), ref0.numpy(), rtol=1e-9, atol=1e-9)
