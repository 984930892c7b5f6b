"""MXFP8 / MXFP4 quantisation (oracle) for the low-precision projections.

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may import it.

[N569] (real-time optimisations) and the single-GPU docs quantise the projections to low-precision
floats; the format here is the OCP microscaling one that gfx950's scaled matrix instructions read:
fp8 e4m3 elements (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; subnormals; largest
finite 448; no infinities) sharing one power-of-two scale per 32 consecutive elements of a row.
Reading (the pages name only the element formats): shared exponent e = floor(log2(amax)) - 8,
8 being the exponent of e4m3's largest power of two, clamped to >= -127 (e8m0 byte e + 127);
elements x / 2^e saturated to +-448 and rounded to nearest, ties to even.

MXFP4 (weights only): fp4 e2m1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; values
0, 0.5, 1, 1.5, 2, 3, 4, 6), the same 32-element blocks and block rule with e2m1's largest exponent 2:
e = floor(log2(amax)) - 2, elements x / 2^e saturated to +-6, nearest with ties to even.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

Array = np.ndarray

E4M3_MAX = 448.0


def round_bf16(x: Array) -> Array:
    """Nearest bfloat16 value of each finite element, in the dtype of x: bfloat16 keeps float32's sign
    and 8 exponent bits and the top 7 of its 23 mantissa bits, so the float32 pattern is rounded on its
    16 low bits, half to even (add 0x7fff plus the lowest kept bit, then clear the 16 low bits)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape).astype(np.asarray(x).dtype)


def e4m3_value(code: Array) -> Array:
    """Real value of e4m3 codes (no NaN codes expected)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e > 0, np.ldexp(1.0 + m / 8.0, e - 7), np.ldexp(m / 8.0, -6))
    return sign * mag


def e4m3_encode(x: Array) -> Array:
    """Round float64 values with |x| <= 448 to e4m3 codes, nearest with ties to even.

    Magnitudes below 2^-6 are on the subnormal grid of spacing 2^-9; above, the grid spacing is
    2^(floor(log2|x|) - 3). The sign bit follows the sign of x (negative zero keeps it).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sub = a < 2.0 ** -6
    e = np.where(sub, -6, np.floor(np.log2(np.where(a > 0, a, 1.0)))).astype(np.int64)
    step = np.ldexp(1.0, np.where(sub, -9, e - 3))
    q = np.rint(a / step)                                   # ties to even
    # sub: code = q (q = 8 is the smallest normal); normal: q in [8, 16], 16 carries into the exponent
    carry = (~sub) & (q == 16)
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    code = np.where(sub, q, ((e + 7) << 3) + (q - 8)).astype(np.int64)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


E2M1_MAX = 6.0


def e2m1_value(code: Array) -> Array:
    """Real value of e2m1 codes (low 4 bits)."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 1
    mag = np.where(e > 0, np.ldexp(1.0 + m / 2.0, e - 1), m / 2.0)
    return sign * mag


def e2m1_encode(x: Array) -> Array:
    """Round float64 values with |x| <= 6 to e2m1 codes, nearest with ties to even: below 1 the grid
    spacing is 1/2 (subnormal 0.5 and zero), above it 2^(floor(log2|x|) - 1)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sub = a < 1.0
    e = np.where(sub, 0, np.floor(np.log2(np.where(a > 0, a, 1.0)))).astype(np.int64)
    step = np.ldexp(1.0, np.where(sub, -1, e - 1))
    q = np.rint(a / step)                                   # ties to even
    # sub: code = q (q = 2 is 1.0, the smallest normal); normal: q in [2, 4], 4 carries into the exponent
    carry = (~sub) & (q == 4)
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 2, q)
    code = np.where(sub, q, ((e + 1) << 1) + (q - 2)).astype(np.int64)
    sign = np.signbit(x).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


_FORMATS = {"e4m3": (8, E4M3_MAX, e4m3_encode, e4m3_value), "e2m1": (2, E2M1_MAX, e2m1_encode, e2m1_value)}


def mx_quantize(x: Array, block: int = 32, fmt: str = "e4m3") -> Tuple[Array, Array]:
    """Quantise the last axis in blocks of ``block``: (element codes, e8m0 scale bytes). e2m1 codes
    are returned one per element (low 4 bits), not packed."""
    emax, vmax, encode, _ = _FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] % block == 0
    xb = x.reshape(x.shape[:-1] + (x.shape[-1] // block, block))
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - emax, -127)
    e = np.maximum(e, -127).astype(np.int64)
    y = np.clip(xb / np.ldexp(1.0, e)[..., None], -vmax, vmax)
    codes = encode(y).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def mx_dequantize(codes: Array, scales: Array, block: int = 32, fmt: str = "e4m3") -> Array:
    v = _FORMATS[fmt][3](codes)
    vb = v.reshape(v.shape[:-1] + (v.shape[-1] // block, block))
    return (vb * np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]).reshape(v.shape)


def mx_linear(a_codes: Array, a_scales: Array, w_codes: Array, w_scales: Array, bias=None, w_fmt: str = "e4m3") -> Array:
    """y = dequant(A) dequant(W)^T (+ b) in float64: what the scaled matrix instruction computes
    before the fp32 rounding of its accumulation (A e4m3; W e4m3 or e2m1)."""
    y = mx_dequantize(a_codes, a_scales) @ mx_dequantize(w_codes, w_scales, fmt=w_fmt).T
    return y if bias is None else y + bias


def relative_error_bound() -> float:
    """Largest relative error of one element in the normal range: half a unit in the last of 3
    mantissa bits."""
    return math.ldexp(1.0, -4)


def mx_attention(q_codes: Array, q_scales: Array, k_codes: Array, k_scales: Array, vt_codes: Array,
                 vt_scales: Array, limits: Array, ref_offset: int = 0) -> Array:
    """Attention on MXFP8 operands with MXFP8 probabilities, per head, in float64.

    [N569] (implementation-level optimisations, mixed precision) keeps the softmax in fp8 e4m3
    beside the fp8 QKV projection. Reading: the probabilities are quantised with the same MX rule
    as the operands, in blocks of 32 consecutive keys of a query's row, before the product with the
    values; the normaliser is the sum of the unquantised probabilities.
      q [H, Lq, d], k [H, Lk, d]: MXFP8 along d (blocks of 32); vt [H, d, Lk]: MXFP8 along keys.
      limits [Lq]: query i sees keys j < limits[i] (a prefix, as the chunk-causal mask gives).
    S = dequant(q) dequant(k)^T / sqrt(d); with M the smallest integer >= every visible S log2(e)
    of the row, p_j = 2^(S_j log2(e) - M) for visible keys, 0 otherwise; l = sum_j p_j;
    o = dequant(mx_quantize(p)) dequant(vt)^T / l  -> [H, Lq, d].
    Scaling p by 2^k (integer k) shifts every block's shared exponent by k and leaves the codes
    alone, so any integer reference gives the same o; ``ref_offset`` adds k to M to show it.
    """
    qd = mx_dequantize(q_codes, q_scales)
    kd = mx_dequantize(k_codes, k_scales)
    vd = mx_dequantize(vt_codes, vt_scales)               # [H, d, Lk_pad]
    H, Lq, d = qd.shape
    Lk = kd.shape[1]
    s = (qd @ np.swapaxes(kd, -1, -2)) * (math.log2(math.e) / math.sqrt(d))   # log2 units
    vis = np.arange(Lk)[None, :] < np.asarray(limits)[:, None]
    s = np.where(vis[None], s, -np.inf)
    with np.errstate(invalid="ignore"):
        m = np.ceil(s.max(axis=-1, keepdims=True))
    m = np.where(np.isfinite(m), m, 0.0) + ref_offset
    p = np.where(vis[None], np.exp2(s - m), 0.0)
    l = p.sum(axis=-1, keepdims=True)
    pad = (-Lk) % 32
    pp = np.concatenate([p, np.zeros((H, Lq, pad))], axis=-1) if pad else p
    pq = mx_dequantize(*mx_quantize(pp))[..., :Lk]
    o = pq @ np.swapaxes(vd[..., :Lk], -1, -2)
    return np.where(l > 0, o / np.where(l > 0, l, 1.0), 0.0)

