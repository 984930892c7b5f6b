"""Pins of the oracle's MXFP8 quantisation against the format's closed forms.

* e4m3 code values: 448 = 1.75 x 2^8 is the largest finite value, 2^-6 the smallest normal, 2^-9
  the smallest subnormal, 1.0 has exponent field 7 (bias 7).
* Every finite code round-trips; midpoints between neighbouring codes go to the even code (ties to
  even), values just above a midpoint go up; encoding is monotone.
* Blocks: the block maximum lands in [256, 448] (the scale is the largest power of two with that
  property, except when saturating above 448); all-zero blocks get code 0 and the smallest scale;
  the dequantised error stays within half a unit in the last place of the element grid.
"""
import numpy as np
import pytest

import oracle as O


def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_e4m3_closed_forms():
    v = O.e4m3_value(np.array([0x7E, 0x08, 0x01, 0x38, 0xB8, 0x00, 0x80, 0x07], dtype=np.uint8))
    assert list(v[:5]) == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0]
    assert v[5] == 0.0 and v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == 7 * 2.0 ** -9                      # largest subnormal


def test_round_trip_ties_and_monotonicity():
    codes = _finite_codes()
    vals = O.e4m3_value(codes)
    np.testing.assert_array_equal(O.e4m3_encode(vals), codes)
    pos = np.sort(O.e4m3_value(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = 0.5 * (pos[:-1] + pos[1:])
    lo_codes = O.e4m3_encode(pos[:-1])
    hi_codes = O.e4m3_encode(pos[1:])
    got = O.e4m3_encode(mids)
    even = np.where(lo_codes % 2 == 0, lo_codes, hi_codes)
    np.testing.assert_array_equal(got, even)
    np.testing.assert_array_equal(O.e4m3_encode(np.nextafter(mids, np.inf)), hi_codes)
    np.testing.assert_array_equal(O.e4m3_encode(np.nextafter(mids, -np.inf)), lo_codes)
    sweep = np.linspace(-448, 448, 20001)
    assert np.all(np.diff(O.e4m3_value(O.e4m3_encode(sweep))) >= 0)


@pytest.mark.parametrize("p", [-20, -3, 0, 5, 40])
def test_block_scale_places_the_maximum(p):
    rng = np.random.default_rng(p + 50)
    x = rng.uniform(-1, 1, (3, 64)) * 2.0 ** p
    x[:, 7] = 2.0 ** p                                  # block 0 maximum is a power of two
    codes, scales = O.mx_quantize(x)
    assert np.all(scales[:, 0] == p - 8 + 127)
    assert np.all(O.e4m3_value(codes[:, 7]) == 256.0)
    y = np.abs(x.reshape(3, 2, 32)) / np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    assert np.all(y.max(axis=-1) >= 256.0) and np.all(y.max(axis=-1) < 512.0)


def test_zero_block_and_error_bound():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((16, 256)) * np.exp(rng.uniform(-8, 8, (16, 1)))
    x[3, 32:64] = 0.0
    codes, scales = O.mx_quantize(x)
    assert scales[3, 1] == 0 and np.all(codes[3, 32:64] == 0)
    xq = O.mx_dequantize(codes, scales)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    y = np.abs(x) / X
    normal = (y >= 2.0 ** -6) & (y <= 448.0)
    assert np.all(np.abs(xq - x)[normal] <= O.mx.relative_error_bound() * np.abs(x)[normal])
    small = y < 2.0 ** -6
    assert np.all(np.abs(xq - x)[small] <= 2.0 ** -10 * X[small])
    over = y > 448.0                                    # saturation to the largest finite value
    assert np.all(np.abs(xq[over]) == 448.0 * X[over])


def test_mx_linear_is_the_product_of_dequantised_operands():
    rng = np.random.default_rng(4)
    a, w = rng.standard_normal((5, 64)), rng.standard_normal((3, 64))
    ac, asc = O.mx_quantize(a)
    wc, wsc = O.mx_quantize(w)
    ref = np.einsum("ik,jk->ij", O.mx_dequantize(ac, asc), O.mx_dequantize(wc, wsc))
    np.testing.assert_allclose(O.mx_linear(ac, asc, wc, wsc), ref, rtol=1e-13, atol=1e-13)
    # quantisation error of the product stays at the element level: ~2^-4 relative per element
    assert np.abs(O.mx_linear(ac, asc, wc, wsc) - a @ w.T).max() < 0.15 * np.abs(a @ w.T).max()


def _proj_inputs(seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((6, 128))
    W = rng.standard_normal((10, 128)) * 0.05
    b = rng.standard_normal(10) * 0.1
    return x, W, b


class _W:
    precision = 1


def test_projection_native_is_linear():
    x, W, b = _proj_inputs()
    class W0:
        precision = 0
    assert np.array_equal(O.project(W0, x, W, b), O.linear(x, W, b))


def test_projection_mx_exact_on_representable_operands():
    """Operands already on the MXFP8 grid (small-integer mantissas, one binade span per block) are
    unchanged by quantisation, so the projection is the plain product."""
    rng = np.random.default_rng(4)
    # multiples of 1/8 up to 14/8 are e4m3 values; with block amax 1.75 the block exponent is -8 and
    # 1.75 * 2^8 = 448, the largest code, so nothing saturates (amax 1.875 would: 480 > 448)
    x = rng.integers(-14, 15, size=(5, 64)) / 8.0
    x[:, ::32] = 1.75
    W = rng.integers(-14, 15, size=(7, 64)) / 4.0
    W[:, ::32] = 3.5
    got = O.project(_W, x, W, None)
    assert np.array_equal(got, x @ W.T)


def test_projection_mx_quantises_along_input_features():
    """Blocks run along the input features of each row: scaling one row of x (or one output row of
    W) by a power of two scales exactly that output row (column) and changes nothing else."""
    x, W, b = _proj_inputs()
    base = O.project(_W, x, W, None)
    x2 = x.copy()
    x2[2] *= 2.0 ** 5
    y2 = O.project(_W, x2, W, None)
    assert np.array_equal(np.delete(y2, 2, axis=0), np.delete(base, 2, axis=0))
    assert np.array_equal(y2[2], base[2] * 2.0 ** 5)
    W2 = W.copy()
    W2[4] *= 2.0 ** -7
    y3 = O.project(_W, x, W2, None)
    assert np.array_equal(np.delete(y3, 4, axis=1), np.delete(base, 4, axis=1))
    assert np.array_equal(y3[:, 4], base[:, 4] * 2.0 ** -7)


def test_projection_mx_error_is_that_of_the_format():
    """Quantising both operands of a 128-term product: relative L2 error of a few percent, between the
    per-element e4m3 bound 2^-4 / sqrt(3)-ish and twice the bound."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 512))
    W = rng.standard_normal((96, 512))
    err = np.linalg.norm(O.project(_W, x, W, None) - x @ W.T) / np.linalg.norm(x @ W.T)
    assert 0.01 < err < 2 * O.relative_error_bound()


# ---- MXFP4 (e2m1 elements) ------------------------------------------------------------------------

E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # the format's eight magnitudes, codes 0..7


def test_e2m1_code_table_and_round_trip():
    codes = np.arange(16)
    vals = O.e2m1_value(codes)
    assert list(vals[:8]) == E2M1_TABLE
    assert list(-vals[8:]) == E2M1_TABLE and all(np.signbit(vals[8:]))
    assert np.array_equal(O.e2m1_encode(vals), codes)


def test_e2m1_ties_to_even_and_nearest():
    # midpoints between neighbours go to the neighbour with an even code (mantissa bit 0)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0])
    assert np.array_equal(O.e2m1_value(O.e2m1_encode(mids)), want)
    assert np.array_equal(O.e2m1_value(O.e2m1_encode(-mids)), -want)
    # just off the midpoints: plain nearest
    eps = 1e-9
    assert np.array_equal(O.e2m1_value(O.e2m1_encode(mids + eps)), np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]))
    assert np.array_equal(O.e2m1_value(O.e2m1_encode(mids - eps)), np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]))


def test_mxfp4_block_rule_and_saturation():
    x = np.zeros((1, 64))
    x[0, 0] = 1.0                                          # amax 1: e = 0 - 2, scaled amax 4 (code 6)
    x[0, 1] = 0.3                                          # 0.3 * 4 = 1.2 -> 1.0
    x[0, 32] = 7.0                                         # amax 7: e = 2 - 2 = 0, 7 > 6 saturates
    x[0, 33] = -2.9                                        # -> -3
    codes, scales = O.mx_quantize(x, fmt="e2m1")
    assert list(scales[0]) == [125, 127]
    assert codes[0, 0] == 6 and codes[0, 1] == 2 and codes[0, 32] == 7 and codes[0, 33] == 13
    back = O.mx_dequantize(codes, scales, fmt="e2m1")
    assert back[0, 0] == 1.0 and back[0, 1] == 0.25 and back[0, 32] == 6.0 and back[0, 33] == -3.0


def test_mxfp4_error_is_that_of_the_format():
    """One mantissa bit: relative error of a normal element at most 1/4 (1.25 -> 1); relative L2 of
    Gaussian blocks between 5% and 20%."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((64, 256))
    codes, scales = O.mx_quantize(x, fmt="e2m1")
    back = O.mx_dequantize(codes, scales, fmt="e2m1")
    err = np.linalg.norm(back - x) / np.linalg.norm(x)
    assert 0.05 < err < 0.2
    # elements at least a quarter of the block maximum sit in e2m1's normal range: error <= 1/4
    xb = x.reshape(64, 8, 32)
    big = np.abs(xb) >= np.abs(xb).max(axis=-1, keepdims=True) / 4
    bb = back.reshape(64, 8, 32)
    sat = np.abs(xb) > 6 * np.ldexp(1.0, scales.astype(int) - 127)[..., None]
    rel = np.abs(bb - xb) / np.abs(xb)
    assert rel[big & ~sat].max() <= 0.25 + 1e-12


def test_projection_mxfp4_weights():
    """Precision 2: activations MXFP8, weights MXFP4 -- the plain product of the two dequantised operands."""
    class W2:
        precision = 2
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 64))
    W = rng.standard_normal((7, 64))
    xc, xs = O.mx_quantize(O.round_bf16(x))   # the activations enter as their bf16 rows
    wc, ws = O.mx_quantize(W, fmt="e2m1")
    want = O.mx_dequantize(xc, xs) @ O.mx_dequantize(wc, ws, fmt="e2m1").T
    assert np.array_equal(O.project(W2, x, W, None), want)


def test_projection_mx_reads_bf16_rows():
    """The low-precision projection quantises the bf16 value of each activation: inputs that differ
    only below bf16's precision give the same product, and the product equals the one of the rounded
    input."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    W = rng.standard_normal((9, 128)) * 0.05
    xr = O.round_bf16(x)
    nudge = (xr * np.float32(2.0 ** -12)).astype(np.float32)   # well inside half a bf16 step of xr
    assert np.array_equal(O.round_bf16(xr + nudge), xr)
    assert np.array_equal(O.project(_W, x, W, None), O.project(_W, xr, W, None))
    assert np.array_equal(O.project(_W, xr + nudge, W, None), O.project(_W, xr, W, None))


def test_round_bf16_is_round_to_nearest_even():
    """Against the library conversion (torch, float32 -> bfloat16 -> float32, round to nearest even) on
    random values over many binades, exact halfway patterns (ties go to the even neighbour) and signed
    zeros and subnormals."""
    import torch
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(4096) * np.exp2(rng.integers(-60, 60, 4096))).astype(np.float32)
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000, 0x00018000, 0x7F7F8000 - 0x10000],
                    dtype=np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, 1e-40, -1e-40, 1.0, -3.5], dtype=np.float32)
    for v in (x, ties, special):
        want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(O.round_bf16(v).view(np.uint32), want.view(np.uint32))
    # the halfway cases land on the even neighbour: 1 + 2^-8 -> 1, (1 + 2^-7) + 2^-8 -> 1 + 2^-6
    assert O.round_bf16(np.float32(1 + 2.0 ** -8)) == np.float32(1.0)
    assert O.round_bf16(np.float32(1 + 2.0 ** -7 + 2.0 ** -8)) == np.float32(1 + 2.0 ** -6)


# ---- MXFP8 attention (probabilities quantised in blocks of 32 keys) ----------------------------------

def _mx_attn_inputs(H, Lq, Lk, d, seed, qscale=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, Lq, d)) * qscale
    k = rng.standard_normal((H, Lk, d))
    v = rng.standard_normal((H, Lk, d))
    pad = (-Lk) % 64
    vt = np.concatenate([np.swapaxes(v, 1, 2), np.zeros((H, d, pad))], axis=-1)
    return O.mx_quantize(q), O.mx_quantize(k), O.mx_quantize(vt)


def test_mx_attention_uniform_scores_average_the_values():
    """Zero queries: every visible key scores 0, each probability is exactly 1 (representable), so
    the output is the plain mean of the visible dequantised values."""
    (qc, qs), kq, vq = _mx_attn_inputs(2, 5, 70, 64, 1)
    qc = np.zeros_like(qc)
    limits = np.array([1, 17, 32, 33, 70])
    o = O.mx_attention(qc, qs, *kq, *vq, limits)
    vd = O.mx_dequantize(*vq)
    for i, lim in enumerate(limits):
        np.testing.assert_allclose(o[:, i], vd[:, :, :lim].mean(axis=-1), rtol=1e-13, atol=1e-13)


def test_mx_attention_dominant_key():
    """One key far above the others (2^-40 and below after the reference): the output is that key's
    value row times one common factor q(p)/p, the rounding of its probability over the unquantised
    normaliser, within e4m3's 2^-4; the rest reaches it only through probabilities below 2^-40."""
    H, Lk, d = 1, 96, 64
    rng = np.random.default_rng(2)
    k = rng.standard_normal((H, Lk, d)) * 0.01
    k[0, 37] = 1.0
    q = np.full((H, 1, d), 4.0)      # score of key 37: 4 d / sqrt(d) = 32; log2 units 46
    vt = rng.standard_normal((H, d, Lk))
    o = O.mx_attention(*O.mx_quantize(q), *O.mx_quantize(k), *O.mx_quantize(vt), np.array([Lk]))
    v37 = O.mx_dequantize(*O.mx_quantize(vt))[0, :, 37]
    c = o[0, 0] @ v37 / (v37 @ v37)
    assert abs(c - 1.0) <= 2.0 ** -4 and c != 1.0
    np.testing.assert_allclose(o[0, 0], c * v37, rtol=0, atol=1e-9 * np.abs(v37).max())


def test_mx_attention_integer_reference_is_irrelevant():
    """Probabilities scaled by 2^k quantise to the same codes with shifted block exponents, so the
    output does not depend on the integer reference: equal up to exp2's own rounding (a different
    argument), far below the 2^-4 steps a changed code would make."""
    qq, kq, vq = _mx_attn_inputs(3, 9, 100, 128, 3, qscale=2.0)
    limits = np.array([3, 10, 31, 32, 33, 64, 65, 99, 100])
    o0 = O.mx_attention(*qq, *kq, *vq, limits)
    for off in (-3, 1, 7):
        np.testing.assert_allclose(O.mx_attention(*qq, *kq, *vq, limits, ref_offset=off), o0, rtol=1e-12, atol=1e-14)
    pc, ps = O.mx_quantize(np.random.default_rng(4).random((5, 64)))
    pc2, ps2 = O.mx_quantize(np.ldexp(O.mx_dequantize(pc, ps), -5))
    assert np.array_equal(pc2, pc) and np.array_equal(ps2.astype(int), ps.astype(int) - 5)


@pytest.mark.parametrize("Lk", [32, 77, 130])
def test_mx_attention_within_the_probability_rounding_bound(Lk):
    """Against exact attention on the same dequantised operands (the model's attention function with
    the prefix mask). With the block scale 2^e (e = floor(log2 of the block's largest probability)
    - 8) an e4m3 probability is off by at most: half a unit in its last place, 2^-4 of itself, in
    the normal range; p - 448 2^e where the block's top values saturate at 448; 2^-10 2^e (half
    the subnormal step) below the normal range. So |o - o_exact| <= sum_j b_j |v_j| / l per
    output element, b_j = max(2^-4 p_j, p_j - 448 2^e) + 2^-10 2^e."""
    H, Lq, d = 2, 7, 64
    qq, kq, vq = _mx_attn_inputs(H, Lq, Lk, d, 10 + Lk, qscale=1.5)
    limits = np.minimum(np.array([1, 5, 31, 32, 33, 60, Lk]), Lk)
    o = O.mx_attention(*qq, *kq, *vq, limits)
    qd, kd = O.mx_dequantize(*qq), O.mx_dequantize(*kq)
    vd = np.swapaxes(O.mx_dequantize(*vq)[..., :Lk], 1, 2)          # [H, Lk, d]
    vis = np.arange(Lk)[None, :] < limits[:, None]
    exact = O.attention(qd, kd, vd, vis)
    # probabilities on the oracle's own scale: 2^(S log2 e - M), M the row's ceiling in log2 units
    s = qd @ np.swapaxes(kd, 1, 2) * (np.log2(np.e) / np.sqrt(d))
    s = np.where(vis[None], s, -np.inf)
    p = np.where(vis[None], np.exp2(s - np.ceil(s.max(axis=-1, keepdims=True))), 0.0)
    l = p.sum(axis=-1, keepdims=True)
    pad = (-Lk) % 32
    pb = np.concatenate([p, np.zeros((H, Lq, pad))], axis=-1).reshape(H, Lq, -1, 32).max(axis=-1)
    pmax = np.repeat(pb, 32, axis=-1)[..., :Lk]
    scale = np.ldexp(1.0, (np.floor(np.log2(np.where(pmax > 0, pmax, 1.0))) - 8).astype(int))
    b = np.maximum(2.0 ** -4 * p, p - 448 * scale) + 2.0 ** -10 * scale
    bound = (b @ np.abs(vd)) / l
    err = np.abs(o - exact)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-15)
    assert err.max() > 0          # the probabilities really are rounded
