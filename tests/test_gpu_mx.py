"""MXFP8 projections through the C ABI (wam_mx_quantize, wam_op_linear_mx) against oracle/mx.py.

* Quantisation is integer work on exactly representable inputs (bf16 or fp32 values, power-of-two
  scaling): codes and scale bytes must match the oracle bit for bit.
* The product: every e4m3 x e4m3 product times its two power-of-two scales is exact, but the scaled
  matrix instruction sums the products of 8 consecutive k after aligning them to the largest one and
  cutting each toward zero 13 bits below it (measured with rows of known exact sums: 256 + 2^-5 is
  kept, 256 + 2^-6 is not, 256 - 2^-6 gives 256; terms 8 apart are not aligned together). So per
  group of 8 the error is below 8 * 2^-12 * max|p| = 2^-9 max|p|, and the group sums then go through
  fp32 additions (at most K/8, each within 2^-23 of the running sum). With G = sum over groups of
  max|a| max|w| and S = sum |a w|, the accumulation error is below t = 2^-9 G + (K/8) 2^-23 S; the
  bf16 output adds 2^-8 (|ref| + t). The test checks that element bound and a relative L2 error of at
  most 1e-2, which a wrong scale byte or k order exceeds many times over.
* Operand codes for the product tests are drawn directly (uniform bytes, NaN codes excluded) with
  scale exponents in [-4, 4]; the end-to-end test quantises seeded bf16 activations and weights on
  both sides independently.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import world_action_video_amd as wam
from world_action_video_amd.device import to_device

pytestmark = pytest.mark.gpu


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def key(name):
    return synth.tensor_key(101, 0, name)


def draw(shape, name, sigma=1.0):
    return synth.fill(shape, key(name), "normal", sigma=sigma)


def draw_codes(rows, cols, name):
    """Uniform e4m3 codes (0x7f / 0xff, the NaN codes, replaced by 0x7e / 0xfe) and scale bytes
    127 + [-4, 4]."""
    u = synth.uniform01(rows * cols, key(name + "_c"))
    codes = np.floor(u * 256).astype(np.uint8).reshape(rows, cols)
    codes[(codes & 0x7F) == 0x7F] -= 1
    s = synth.uniform01(rows * cols // 32, key(name + "_s"))
    scales = (123 + np.floor(s * 9)).astype(np.uint8).reshape(rows, cols // 32)
    return codes, scales


def dev_u8(a, gpu):
    return torch.from_numpy(np.ascontiguousarray(a)).to(gpu)


def quantise_on_gpu(gpu, x, dtype, ld_pad=0):
    """x: float32 host array (values representable in dtype) -> (codes, scales) host arrays."""
    rows, cols = x.shape
    ld = cols + ld_pad
    xp = np.zeros((rows, ld), dtype=np.float32)
    xp[:, :cols] = x
    X = to_device(xp, dtype, gpu)
    ldq = cols + 16
    codes = torch.full((rows, ldq), 0x5A, dtype=torch.uint8, device=gpu)
    scales = torch.full((rows, cols // 32), 0x5A, dtype=torch.uint8, device=gpu)
    wam.wam_mx_quantize(wam.WAM_BF16 if dtype == "bf16" else wam.WAM_F32, X, ld, rows, cols, codes, ldq, scales)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    assert np.all(c[:, cols:] == 0x5A), "row padding written"
    return c[:, :cols], scales.cpu().numpy()


def special_rows(cols):
    """Rows with the edge cases of the encoding, one 32-block each, repeated to ``cols``."""
    blocks = []
    b = np.zeros(32)
    blocks.append(b.copy())                                   # zero block: scale byte 0, codes 0
    b = np.zeros(32)
    b[::2] = -0.0
    blocks.append(b)                                          # negative zeros keep their sign
    b = np.full(32, 0.5)
    b[0] = 256.0                                              # amax a power of two: e = 0
    b[1:9] = [1.0625, 1.1875, -1.0625, 2.125, 0.0009765625, 0.0029296875, 480.0 / 2, 3.0 * 2 ** -10]
    blocks.append(b)                                          # ties to even, subnormal ties
    b = np.linspace(-1.0, 1.0, 32) * 510.0                   # amax 510: e = 0, |x| > 448 saturates
    blocks.append(b)
    b = np.linspace(-1.0, 1.0, 32) * 2.0 ** 40                # large exponent
    blocks.append(b)
    b = np.linspace(-1.0, 1.0, 32) * 2.0 ** -100              # small exponent: e = -108
    blocks.append(b)
    b = np.linspace(-1.0, 1.0, 32) * 2.0 ** -120              # e clamps at -127 (scaled values < 2^9)
    blocks.append(b)
    row = np.concatenate(blocks * (cols // (32 * len(blocks)) + 1))[:cols]
    return np.stack([row, -row, np.roll(row, 32)]).astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,ld_pad", [(1, 32, 0), (67, 256, 8), (300, 1024, 0), (5, 5120, 16)])
def test_mx_quantize_bit_exact(gpu, dtype, rows, cols, ld_pad):
    print("mx_quantize", dtype, rows, cols, ld_pad, flush=True)
    x = draw((rows, cols), "q%d_%d" % (rows, cols))
    # give the row blocks different magnitudes (2^-12 .. 2^12)
    mag = np.ldexp(1.0, (np.arange(rows * (cols // 32)) % 25 - 12)).reshape(rows, cols // 32)
    x = (x.reshape(rows, cols // 32, 32) * mag[..., None]).reshape(rows, cols).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_bf16(x)
    codes, scales = quantise_on_gpu(gpu, x, dtype, ld_pad)
    rc, rs = O.mx_quantize(x.astype(np.float64))
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mx_quantize_special_blocks(gpu, dtype):
    x = special_rows(448)
    if dtype == "bf16":
        x = synth.round_bf16(x)
    codes, scales = quantise_on_gpu(gpu, x, dtype)
    rc, rs = O.mx_quantize(x.astype(np.float64))
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


def acc_bound(da, dw):
    """t = 2^-9 G + (K/8) 2^-23 S for dequantised operands da [M][K], dw [N][K]."""
    K = da.shape[1]
    ag = np.abs(da).reshape(da.shape[0], K // 8, 8).max(axis=2)
    wg = np.abs(dw).reshape(dw.shape[0], K // 8, 8).max(axis=2)
    G = ag @ wg.T
    S = np.abs(da) @ np.abs(dw).T
    return 2.0 ** -9 * G + (K / 8) * 2.0 ** -23 * S


def _tolerance(ref_pre, t, act):
    """Element bound: accumulation bound t through the activation, then bf16 rounding.

    An error t before the activation moves its output by at most L t, L the activation's largest
    slope: GELU-tanh's derivative lies in [-0.129, 1.129] (maximum at x = 1.42), so L = 1.13; SiLU's in
    [-0.0998, 1.0998] (maximum at x = 2.40), so L = 1.1. For SwiGLU pairs SiLU(g) u the product rule
    adds |u| L t_g + |SiLU(g)| t_u + L t_g t_u."""
    if act == 0:
        ref = ref_pre
        return ref, 2.0 ** -8 * (np.abs(ref) + t) + t
    if act == 1:
        ref = O.gelu_tanh(ref_pre)
        return ref, 2.0 ** -8 * (np.abs(ref) + 1.13 * t) + 1.13 * t
    g, u = ref_pre[:, 0::2], ref_pre[:, 1::2]
    tg, tu = t[:, 0::2], t[:, 1::2]
    ref = O.silu(g) * u
    tt = 1.1 * np.abs(u) * tg + np.abs(O.silu(g)) * tu + 1.1 * tg * tu
    return ref, 2.0 ** -8 * (np.abs(ref) + tt) + tt


def _check_bound(out, ref, tol, t=None):
    bad = ~(np.abs(out - ref) <= tol)
    if bad.any():
        idx = np.argwhere(bad)
        print("%d of %d outside the bound; first:" % (len(idx), out.size), flush=True)
        for r, c in idx[:12]:
            print("  [%d, %d] out %r ref %r tol %r t %r" % (r, c, float(out[r, c]), float(ref[r, c]), float(tol[r, c]),
                                                         None if t is None else float(t[r, c])), flush=True)
        rows, cols = np.unique(idx[:, 0]), np.unique(idx[:, 1])
        print("  rows", rows[:40], "cols", cols[:40], flush=True)
    assert not bad.any()


def _run_mx(gpu, ac, as_, wc, ws_, b, act, split, M, N, K):
    A, AS, W, WS = dev_u8(ac, gpu), dev_u8(as_, gpu), dev_u8(wc, gpu), dev_u8(ws_, gpu)
    B = torch.from_numpy(b).to(gpu) if b is not None else None
    C = torch.full((M, N // 2 if act == 2 else N), float("nan"), dtype=torch.bfloat16, device=gpu)
    ws = torch.empty(4 * M * N * 4, dtype=torch.uint8, device=gpu) if split else None
    wam.wam_op_linear_mx(A, AS, K, W, WS, K, B, C, C.shape[1], M, N, K, act, ws=ws)
    torch.cuda.synchronize()
    return C.float().cpu().numpy()


MX_CASES = [(1, 64, 128), (67, 200, 128), (300, 384, 512), (928, 1024, 256), (130, 96, 1024), (257, 260, 2048),
            (260, 516, 384), (928, 512, 5120)]


@pytest.mark.parametrize("M,N,K", MX_CASES)
@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("split", [False, True])
def test_op_linear_mx(gpu, M, N, K, act, split):
    """With a workspace, products of fewer than 128 256x256 tiles split over K (tiles of 128 k)."""
    print("linear_mx", M, N, K, act, split, flush=True)
    ac, as_ = draw_codes(M, K, "a%d_%d_%d" % (M, N, K))
    wc, ws_ = draw_codes(N, K, "w%d_%d_%d" % (M, N, K))
    if act == 2 and (N // 2) % 4:   # the output row pitch N/2 must be a multiple of 4: rejected, nothing written
        with pytest.raises(wam.WamError, match="ldc"):
            _run_mx(gpu, ac, as_, wc, ws_, None, act, split, M, N, K)
        return
    if act == 1:   # scale exponent -7: GELU's argument stays within a few units of zero
        as_ = np.minimum(as_, 120).astype(np.uint8)
    da, dw = O.mx_dequantize(ac, as_), O.mx_dequantize(wc, ws_)
    pre = da @ dw.T
    b = (draw((N,), "b%d" % N) * np.sqrt(np.mean(pre ** 2))).astype(np.float32)   # bias as large as the product
    out = _run_mx(gpu, ac, as_, wc, ws_, b, act, split, M, N, K)
    pre = pre + b
    t = acc_bound(da, dw)
    ref, tol = _tolerance(pre, t, act)
    _check_bound(out, ref, tol, t if act == 0 else None)
    assert rel_l2(out, ref) <= 1e-2


def test_op_linear_mx_matches_oracle_product_no_bias(gpu):
    M, N, K = 300, 256, 640
    ac, as_ = draw_codes(M, K, "nb_a")
    wc, ws_ = draw_codes(N, K, "nb_w")
    out = _run_mx(gpu, ac, as_, wc, ws_, None, 0, False, M, N, K)
    ref = O.mx_linear(ac, as_, wc, ws_)
    t = acc_bound(O.mx_dequantize(ac, as_), O.mx_dequantize(wc, ws_))
    _check_bound(out, ref, 2.0 ** -8 * (np.abs(ref) + t) + t, t)


def test_op_linear_mx_deterministic(gpu):
    M, N, K = 928, 1024, 2048
    ac, as_ = draw_codes(M, K, "det_a")
    wc, ws_ = draw_codes(N, K, "det_w")
    b = draw((N,), "det_b", 1.0)
    for split in (False, True):
        o1 = _run_mx(gpu, ac, as_, wc, ws_, b, 0, split, M, N, K)
        o2 = _run_mx(gpu, ac, as_, wc, ws_, b, 0, split, M, N, K)
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


@pytest.mark.parametrize("M,N,K", [(928, 15360, 5120), (928, 5120, 13824), (464, 27648, 5120)])
def test_op_linear_mx_full_size_end_to_end(gpu, M, N, K):
    """Block-sized projections: bf16 activations and weights quantised on each side independently,
    then the product; rows sampled for the oracle (all columns of 48 rows, ragged last tile
    included). Also bounds the MXFP8 error against the unquantised bf16 product."""
    print("linear_mx full", M, N, K, flush=True)
    x = synth.round_bf16(draw((M, K), "e2e_x%d_%d" % (M, K)))
    w = synth.round_bf16(draw((N, K), "e2e_w%d_%d" % (N, K), 0.02))
    b = draw((N,), "e2e_b%d" % N, 0.02)
    X, W = to_device(x, "bf16", gpu), to_device(w, "bf16", gpu)
    AQ = torch.empty((M, K), dtype=torch.uint8, device=gpu)
    AS = torch.empty((M, K // 32), dtype=torch.uint8, device=gpu)
    WQ = torch.empty((N, K), dtype=torch.uint8, device=gpu)
    WS = torch.empty((N, K // 32), dtype=torch.uint8, device=gpu)
    wam.wam_mx_quantize(wam.WAM_BF16, X, K, M, K, AQ, K, AS)
    wam.wam_mx_quantize(wam.WAM_BF16, W, K, N, K, WQ, K, WS)
    Bt = torch.from_numpy(b).to(gpu)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
    wam.wam_op_linear_mx(AQ, AS, K, WQ, WS, K, Bt, C, N, M, N, K, 0)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 40)), np.arange(M - 8, M)]))
    out = C.float().cpu().numpy()[rows]
    rc, rs = O.mx_quantize(x[rows].astype(np.float64))
    wc, wsc = O.mx_quantize(w.astype(np.float64))
    ref = O.mx_linear(rc, rs, wc, wsc, b)
    t = acc_bound(O.mx_dequantize(rc, rs), O.mx_dequantize(wc, wsc))
    _check_bound(out, ref, 2.0 ** -8 * (np.abs(ref) + t) + t, t)
    assert rel_l2(out, ref) <= 1e-2
    exact = x[rows].astype(np.float64) @ w.astype(np.float64).T + b
    err = rel_l2(out, exact)
    print("MXFP8 relative L2 against the unquantised product: %.4f" % err, flush=True)
    assert err <= 0.06


def test_op_linear_mx_exact_sum_rows(gpu):
    """Rows with known exact sums (W = 1.0): tiny terms beside a large one in the same group of 8 k
    (the adversarial case of the accumulation bound), in other groups, blocks and k-tiles, with
    cancellation and with scale exponents 2^+-10. Each result must lie within the bound t of the
    exact sum; terms in separate groups must come out exact."""
    M, N, K = 64, 256, 512
    a = np.zeros((M, K))
    asc = np.full((M, K // 32), 127, np.uint8)
    rows = [
        ([(0, 256.0), (1, 2.0 ** -6)], False), ([(0, 256.0), (1, 2.0 ** -5)], True),
        ([(0, 256.0), (1, -2.0 ** -6)], False), ([(0, 448.0), (1, -448.0), (2, 2.0 ** -9)], False),
        ([(0, 256.0), (8, 2.0 ** -6)], True), ([(0, 256.0), (40, 2.0 ** -6)], True),
        ([(0, 256.0), (64, 2.0 ** -9)], True), ([(0, 256.0), (128, 2.0 ** -6)], True),
        ([(0, 448.0)] + [(k, 0.1171875) for k in range(1, 32)], False),
        ([(0, 1.0)] + [(k, 2.0 ** -9) for k in range(1, 32)], True), ([(0, 2.0 ** -9)], True),
    ]
    for r, (terms, _) in enumerate(rows):
        for k, v in terms:
            a[r, k] = v
    r_sc = len(rows)   # 2^10 + 2^-10 through the block scales
    a[r_sc, 0] = a[r_sc, 32] = 1.0
    asc[r_sc, 0], asc[r_sc, 1] = 137, 117
    ac = O.e4m3_encode(a)
    assert np.array_equal(O.e4m3_value(ac), a)
    wc = np.full((N, K), 0x38, np.uint8)
    wsc = np.full((N, K // 32), 127, np.uint8)
    A, AS, W, WS = [dev_u8(v, gpu) for v in (ac, asc, wc, wsc)]
    C = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
    part = torch.zeros(4 * M * N, dtype=torch.float32, device=gpu)   # K = 512, one tile: 2 splits of 256 k
    wam.wam_op_linear_mx(A, AS, K, W, WS, K, None, C, N, M, N, K, 0, ws=part)
    torch.cuda.synchronize()
    p = part.cpu().numpy()[:2 * M * N].reshape(2, M, N).astype(np.float64)
    got = p[0] + p[1]
    da, dw = O.mx_dequantize(ac, asc), O.mx_dequantize(wc, wsc)
    ex = da @ dw.T
    t = acc_bound(da, dw)
    assert np.all(np.abs(got - ex) <= t)
    for r, (_, exact) in enumerate(rows + [(None, True)]):
        assert np.all(got[r] == got[r, 0])
        if exact:
            assert got[r, 0] == ex[r, 0], (r, got[r, 0], ex[r, 0])


# ---- MXFP4 weights (e2m1 codes, two per byte, low nibble first) -----------------------------------

def unpack_e2m1(packed, cols):
    p = np.asarray(packed, dtype=np.uint8)[:, :cols // 2]
    out = np.empty((p.shape[0], cols), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def pack_e2m1(codes):
    c = np.asarray(codes, dtype=np.uint8)
    return np.ascontiguousarray((c[:, 0::2] & 0xF) | ((c[:, 1::2] & 0xF) << 4))


def quantise4_on_gpu(gpu, x, dtype):
    rows, cols = x.shape
    X = to_device(np.ascontiguousarray(x, dtype=np.float32), dtype, gpu)
    ldq = cols // 2 + 16
    codes = torch.full((rows, ldq), 0x5A, dtype=torch.uint8, device=gpu)
    scales = torch.full((rows, cols // 32), 0x5A, dtype=torch.uint8, device=gpu)
    wam.wam_mx4_quantize(wam.WAM_BF16 if dtype == "bf16" else wam.WAM_F32, X, cols, rows, cols, codes, ldq, scales)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    assert np.all(c[:, cols // 2:] == 0x5A), "row padding written"
    return unpack_e2m1(c, cols), scales.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(1, 32), (67, 256), (300, 1024), (5, 5120)])
def test_mx4_quantize_bit_exact(gpu, dtype, rows, cols):
    print("mx4_quantize", dtype, rows, cols, flush=True)
    x = draw((rows, cols), "q4_%d_%d" % (rows, cols))
    mag = np.ldexp(1.0, (np.arange(rows * (cols // 32)) % 25 - 12)).reshape(rows, cols // 32)
    x = (x.reshape(rows, cols // 32, 32) * mag[..., None]).reshape(rows, cols).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_bf16(x)
    codes, scales = quantise4_on_gpu(gpu, x, dtype)
    rc, rs = O.mx_quantize(x.astype(np.float64), fmt="e2m1")
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mx4_quantize_special_blocks(gpu, dtype):
    """Zero and negative-zero blocks, every e2m1 midpoint (ties to even), saturation above 6, large and
    small exponents."""
    blocks = [np.zeros(32), np.where(np.arange(32) % 2 == 0, -0.0, 0.0)]
    b = np.full(32, 0.5)
    b[0] = 4.0                                                   # amax 4: e = 0, scaled = x
    b[1:15] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, 0.3, 3.4]
    blocks.append(b)
    b = np.linspace(-1.0, 1.0, 32) * 7.5                         # amax 7.5: e = 0, |x| > 6 saturates
    blocks.append(b)
    b = np.full(32, 1.0)
    b[3] = 5.0                                                   # tie 5 -> 4 with amax 5 (e = 0)
    blocks.append(b)
    blocks.append(np.linspace(-1.0, 1.0, 32) * 2.0 ** 40)
    blocks.append(np.linspace(-1.0, 1.0, 32) * 2.0 ** -120)
    row = np.concatenate(blocks)
    x = np.stack([row, -row, np.roll(row, 32)]).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_bf16(x)
    codes, scales = quantise4_on_gpu(gpu, x, dtype)
    rc, rs = O.mx_quantize(x.astype(np.float64), fmt="e2m1")
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rc)


def draw_codes4(rows, cols, name):
    u = synth.uniform01(rows * cols, key(name + "_c4"))
    codes = np.floor(u * 16).astype(np.uint8).reshape(rows, cols)
    s = synth.uniform01(rows * cols // 32, key(name + "_s4"))
    scales = (123 + np.floor(s * 9)).astype(np.uint8).reshape(rows, cols // 32)
    return codes, scales


@pytest.mark.parametrize("M,N,K", MX_CASES)
@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("split", [False, True])
def test_op_linear_mx4(gpu, M, N, K, act, split):
    """MXFP8 activations times MXFP4 weights, same bound as the MXFP8 product (the fp8 x fp4 products
    are exact; the accumulation is the same instruction's)."""
    if act == 2 and (N // 2) % 4:
        pytest.skip("SwiGLU output pitch N/2 must be a multiple of 4 (rejection covered by the MXFP8 test)")
    print("linear_mx4", M, N, K, act, split, flush=True)
    ac, as_ = draw_codes(M, K, "a4%d_%d_%d" % (M, N, K))
    wc, ws_ = draw_codes4(N, K, "w4%d_%d_%d" % (M, N, K))
    if act == 1:
        as_ = np.minimum(as_, 120).astype(np.uint8)
    da, dw = O.mx_dequantize(ac, as_), O.mx_dequantize(wc, ws_, fmt="e2m1")
    pre = da @ dw.T
    b = (draw((N,), "b4%d" % N) * np.sqrt(np.mean(pre ** 2))).astype(np.float32)
    A, AS, W, WS = dev_u8(ac, gpu), dev_u8(as_, gpu), dev_u8(pack_e2m1(wc), gpu), dev_u8(ws_, gpu)
    B = torch.from_numpy(b).to(gpu)
    C = torch.full((M, N // 2 if act == 2 else N), float("nan"), dtype=torch.bfloat16, device=gpu)
    wsb = torch.empty(4 * M * N * 4, dtype=torch.uint8, device=gpu) if split else None
    wam.wam_op_linear_mx(A, AS, K, W, WS, K // 2, B, C, C.shape[1], M, N, K, act, ws=wsb, w_format=wam.WAM_MX_E2M1)
    torch.cuda.synchronize()
    out = C.float().cpu().numpy()
    pre = pre + b
    t = acc_bound(da, dw)
    ref, tol = _tolerance(pre, t, act)
    _check_bound(out, ref, tol, t if act == 0 else None)
    assert rel_l2(out, ref) <= 1e-2


def test_op_linear_mx4_full_size_end_to_end(gpu):
    """928 x 15360 x 5120 (QKV shape): bf16 activations quantised to MXFP8 and bf16 weights to MXFP4 on
    each side independently, rows sampled; and the MXFP4-weight error against the unquantised product."""
    M, N, K = 928, 15360, 5120
    x = synth.round_bf16(draw((M, K), "e2e4_x"))
    w = synth.round_bf16(draw((N, K), "e2e4_w", 0.02))
    X, Wt = to_device(x, "bf16", gpu), to_device(w, "bf16", gpu)
    AQ = torch.empty((M, K), dtype=torch.uint8, device=gpu)
    AS = torch.empty((M, K // 32), dtype=torch.uint8, device=gpu)
    WQ = torch.empty((N, K // 2), dtype=torch.uint8, device=gpu)
    WS = torch.empty((N, K // 32), dtype=torch.uint8, device=gpu)
    wam.wam_mx_quantize(wam.WAM_BF16, X, K, M, K, AQ, K, AS)
    wam.wam_mx4_quantize(wam.WAM_BF16, Wt, K, N, K, WQ, K // 2, WS)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
    wam.wam_op_linear_mx(AQ, AS, K, WQ, WS, K // 2, None, C, N, M, N, K, 0, w_format=wam.WAM_MX_E2M1)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, 29), np.arange(M - 4, M)]))
    out = C.float().cpu().numpy()[rows]
    rc, rs = O.mx_quantize(x[rows].astype(np.float64))
    wc, wsc = O.mx_quantize(w.astype(np.float64), fmt="e2m1")
    ref = O.mx_linear(rc, rs, wc, wsc, w_fmt="e2m1")
    t = acc_bound(O.mx_dequantize(rc, rs), O.mx_dequantize(wc, wsc, fmt="e2m1"))
    _check_bound(out, ref, 2.0 ** -8 * (np.abs(ref) + t) + t, t)
    exact = x[rows].astype(np.float64) @ w.astype(np.float64).T
    err = rel_l2(out, exact)
    print("MXFP4-weight relative L2 against the unquantised product: %.4f" % err, flush=True)
    assert err <= 0.2
