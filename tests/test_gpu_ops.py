"""Kernel-level parity through the C ABI (wam_op_linear, wam_op_attention, wam_op_split_finish,
wam_op_modulated_norm, wam_op_qkv_cache) against the oracle.

Inputs are seeded synth draws (bf16-representable), identical on both sides. Tolerances:
* linear, bf16: fp32 accumulation of exact bf16 products, then one rounding of the output to bf16,
  so |gpu - ref| <= 2^-8 |ref| + 2^-8 * 1e-2 (a bf16 half-ulp, plus slack for the summation order);
* linear, fp32: relative L2 <= 1e-5 (fp32 summation of K products);
* attention, bf16: probabilities enter the second product rounded to bf16 and the output is
  rounded to bf16: relative L2 <= 1e-2; fp32: relative L2 <= 1e-5.
"""
import math

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


def draw(shape, name, sigma=1.0):
    return synth.fill(shape, synth.tensor_key(100, 0, name), "normal", sigma=sigma)


def host(t):
    return t.float().cpu().numpy()


LINEAR_CASES = [(1, 64, 64), (67, 200, 128), (300, 384, 512), (928, 1024, 256), (130, 96, 1024), (300, 520, 1024),
                (257, 260, 2048), (260, 258, 192),
                (520, 16380, 320),    # 192 tiles of 256 x 256 -> 222 of 256 x 224 (ragged M and N)
                (1024, 16384, 128)]   # 256 tiles of 256 x 256 (one round) against 312 of 192 x 320


def split_ws(gpu, M, N):
    """Scratch for up to four split-K partial products of an [M][N] output."""
    return torch.empty(4 * M * N * 4 + 256, dtype=torch.uint8, device=gpu)[:4 * M * N * 4]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("split", [False, True])
def test_op_linear_small(gpu, dtype, M, N, K, act, split):
    """bf16 products with M, N >= 256 take the four-wave tiles (192 x 320 for most of these shapes,
    256 x 256 for the last, 256 x 224 for the wide one); with a workspace, those of fewer than 128
    tiles split over K."""
    if split and dtype == "f32":
        pytest.skip("split-K serves the bf16 path only")
    print("linear", dtype, M, N, K, act, split, flush=True)
    a = draw((M, K), "a%d_%d_%d" % (M, N, K))
    w = draw((N, K), "w%d_%d_%d" % (M, N, K), 0.05)
    b = draw((N,), "b%d" % N, 0.1)
    ref = a.astype(np.float64) @ w.astype(np.float64).T + b
    if act == 1:
        ref = O.gelu_tanh(ref)
    elif act == 2:   # SwiGLU pairs: SiLU(gate column 2j) * up column 2j+1
        ref = O.silu(ref[:, 0::2]) * ref[:, 1::2]
    dt = wam.WAM_BF16 if dtype == "bf16" else wam.WAM_F32
    A, W = to_device(a, dtype, gpu), to_device(w, dtype, gpu)
    B = torch.from_numpy(b).to(gpu)
    C = torch.full((M, N // 2 if act == 2 else N), float("nan"), dtype=A.dtype, device=gpu)
    wam.wam_op_linear(dt, A, K, W, K, B, C, C.shape[1], M, N, K, act, ws=split_ws(gpu, M, N) if split else None)
    torch.cuda.synchronize()
    out = host(C)
    if dtype == "bf16":
        assert np.all(np.abs(out - ref) <= np.abs(ref) * 2.0 ** -8 + 2.0 ** -8 * 1e-2)
    else:
        assert rel_l2(out, ref) <= 1e-5


@pytest.mark.parametrize("M,N,K,split", [(928, 15360, 5120, False), (928, 5120, 13824, False), (928, 5120, 13824, True),
                                         (928, 5120, 5120, True), (464, 15360, 5120, True), (1538, 5120, 1536, False),
                                         (2688, 5120, 5120, False)])
def test_op_linear_full_size_sampled(gpu, M, N, K, split):
    _linear_full(gpu, M, N, K, split, 0)


@pytest.mark.parametrize("act", [0, 1])
def test_op_linear_ffn_up_full_size_sampled(gpu, act):
    """FFN-up shape 928 x 13824 x 5120 (256 x 224 tiles: 248 workgroups), plain and with GELU."""
    _linear_full(gpu, 928, 13824, 5120, False, act)


def _linear_full(gpu, M, N, K, split, act):
    """The step's real projection shapes in bf16 (split over K as the block splits them when a
    workspace is given), checked on 4096 sampled outputs computed one by one."""
    print("linear-full", M, N, K, split, act, flush=True)
    a = draw((M, K), "fa%d_%d" % (M, K))
    w = draw((N, K), "fw%d_%d" % (N, K), 0.02)
    b = draw((N,), "fb%d" % N, 0.02)
    A, W = to_device(a, "bf16", gpu), to_device(w, "bf16", gpu)
    B = torch.from_numpy(b).to(gpu)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
    ws = split_ws(gpu, M, N) if split else None
    wam.wam_op_linear(wam.WAM_BF16, A, K, W, K, B, C, N, M, N, K, act, ws=ws)
    torch.cuda.synchronize()
    out = host(C)
    if split:   # the partials are summed in a fixed order: a second run is bit-identical
        C2 = torch.empty_like(C)
        wam.wam_op_linear(wam.WAM_BF16, A, K, W, K, B, C2, N, M, N, K, act, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(C, C2)
    rng = np.random.default_rng(7)
    rows = np.concatenate([rng.integers(0, M, 4000), [0, M - 1] * 48])
    cols = np.concatenate([rng.integers(0, N, 4000), [0, N - 1, N - 1, 0] * 24])
    a_bf = synth.round_bf16(a).astype(np.float64)
    w_bf = synth.round_bf16(w).astype(np.float64)
    ref = np.einsum("ik,ik->i", a_bf[rows], w_bf[cols]) + b[cols]
    if act == 1:
        ref = O.gelu_tanh(ref)
    got = out[rows, cols]
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-3)


def _attn_case(gpu, dtype, br, H, d, Lq, kv_base, chunk_q, kv_total, tag, v_stride=None, ws=None, runs=1):
    k_rows = ((kv_total + 63) // 64) * 64 + 64
    if v_stride is None:
        v_stride = ((kv_total + 63) // 64) * 64
    q = draw((br, H, Lq, d), "q" + tag)
    k = draw((br, H, k_rows, d), "k" + tag)
    v = draw((br, H, kv_total, d), "v" + tag)
    vt = np.zeros((br, H, d, v_stride), np.float32)
    vt[..., :kv_total] = np.swapaxes(v, -1, -2)
    # stale values beyond kv_total must not matter: poison them
    if v_stride > kv_total:
        vt[..., kv_total:] = np.nan
    k[:, :, kv_total:] = np.nan
    Q, K, VT = (to_device(x, dtype, gpu) for x in (q, k, vt))
    dt = wam.WAM_BF16 if dtype == "bf16" else wam.WAM_F32
    outs = []
    for _ in range(runs):
        Ot = torch.full((br * Lq, H * d), float("nan"), dtype=Q.dtype, device=gpu)
        wam.wam_op_attention(dt, Q, K, VT, Ot, br, H, d, Lq, k_rows, v_stride, kv_base, chunk_q, kv_total, ws=ws)
        torch.cuda.synchronize()
        outs.append(host(Ot).reshape(br, Lq, H, d).transpose(0, 2, 1, 3))
    out = outs[0] if runs == 1 else outs
    lim = np.full(Lq, kv_total)
    if chunk_q > 0:
        lim = np.minimum(kv_total, kv_base + (np.arange(Lq) // chunk_q + 1) * chunk_q)
    vis = np.arange(kv_total)[None, :] < lim[:, None]
    ref = np.stack([O.attention(q[b].astype(np.float64), k[b, :, :kv_total].astype(np.float64),
                                v[b].astype(np.float64), vis) for b in range(br)])
    return out, ref


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lq,kv_base,chunk_q,kv_total", [
    (1, 0, 0, 1),            # one key: output = V row
    (5, 0, 0, 9),
    (152, 152, 0, 304),      # tiny workload incremental step
    (304, 0, 152, 304),      # tiny workload full sequence, 2 chunks
    (200, 64, 72, 250),      # ragged chunk-causal
    (130, 0, 0, 769),        # cross-attention length
])
def test_op_attention(gpu, dtype, d, Lq, kv_base, chunk_q, kv_total):
    print("attention", dtype, d, Lq, kv_base, chunk_q, kv_total, flush=True)
    (out, out2), ref = _attn_case(gpu, dtype, 2, 3, d, Lq, kv_base, chunk_q, kv_total,
                                  "%d_%d_%d_%d_%d" % (d, Lq, kv_base, chunk_q, kv_total), runs=2)
    assert np.all(np.isfinite(out))
    assert rel_l2(out, ref) <= (1e-2 if dtype == "bf16" else 1e-5)
    assert np.array_equal(out, out2)   # a second run is bit-identical


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lq,kv_base,chunk_q,kv_total,v_stride", [
    (100, 0, 0, 100, 104),     # value rows shorter than whole 32-key tiles: register-staged kernel
    (130, 0, 0, 769, 776),
    (96, 32, 40, 249, 256),    # rows hold whole tiles: copy kernel, tail keys past kv_total poisoned
])
def test_op_attention_value_row_pitch(gpu, d, Lq, kv_base, chunk_q, kv_total, v_stride):
    """bf16 value rows of tight pitch: both attention kernels (selected by whether a row holds whole
    32-key tiles) against the oracle, with stale keys and values past kv_total set to NaN."""
    print("attention-pitch", d, Lq, kv_base, chunk_q, kv_total, v_stride, flush=True)
    out, ref = _attn_case(gpu, "bf16", 2, 3, d, Lq, kv_base, chunk_q, kv_total, "p%d_%d_%d" % (d, kv_total, v_stride),
                          v_stride=v_stride)
    assert np.all(np.isfinite(out))
    assert rel_l2(out, ref) <= 1e-2


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lq,kv_base,chunk_q,kv_total", [
    (1024, 2053, 0, 3077),     # incremental, ragged last tile
    (1100, 2000, 550, 3100),   # two query chunks over a long cache, chunk-causal
])
def test_op_attention_long_ranges(gpu, d, Lq, kv_base, chunk_q, kv_total):
    """Query and key ranges of the long-context workload's order (1024+ queries over 3072+ keys, many
    tiles per workgroup); one branch and two heads keep the oracle fast."""
    print("attention-long", d, Lq, kv_base, chunk_q, kv_total, flush=True)
    (out, out2), ref = _attn_case(gpu, "bf16", 1, 2, d, Lq, kv_base, chunk_q, kv_total, "l%d_%d_%d" % (d, Lq, kv_total),
                                  runs=2)
    assert np.all(np.isfinite(out))
    assert rel_l2(out, ref) <= 1e-2
    assert np.array_equal(out, out2)   # a second run is bit-identical


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Lq,kv_base,chunk_q,kv_total", [
    (100, 1900, 0, 2000),      # few query blocks over a long cache: eight key ranges
    (512, 0, 64, 512),         # full-sequence chunk-causal: some ranges hold no visible key for some queries
    (300, 1500, 100, 1800),    # chunk-causal over a cache, ragged last tile
])
def test_op_attention_key_split(gpu, d, Lq, kv_base, chunk_q, kv_total):
    """With scratch and few query blocks, bf16 attention splits the keys into ranges and merges them:
    against the oracle, bit-identical across runs, and equal to the unsplit kernel up to rounding."""
    print("attention-split", d, Lq, kv_base, chunk_q, kv_total, flush=True)
    tag = "s%d_%d_%d_%d" % (d, Lq, chunk_q, kv_total)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=gpu)
    (o1, o2), ref = _attn_case(gpu, "bf16", 1, 2, d, Lq, kv_base, chunk_q, kv_total, tag, ws=ws, runs=2)
    plain, _ = _attn_case(gpu, "bf16", 1, 2, d, Lq, kv_base, chunk_q, kv_total, tag)
    assert np.all(np.isfinite(o1))
    assert rel_l2(o1, ref) <= 1e-2
    assert np.array_equal(o1, o2)
    assert rel_l2(o1, plain) <= 1e-2


@pytest.mark.parametrize("H,Lq,kv_base,chunk_q,kv_total", [
    (33, 400, 100, 136, 500),   # chunk-causal over a cache, ragged last block
    (40, 464, 0, 0, 769),       # cross-attention geometry
    (33, 480, 0, 160, 480),     # full-sequence pass of three chunks
    (36, 385, 0, 0, 1000),      # last block of 65 queries: waves 2-4 hold (almost) none
    (40, 400, 0, 0, 20),        # one key tile per block: the single-range five-wave kernel
])
def test_op_attention_five_wave_blocks(gpu, H, Lq, kv_base, chunk_q, kv_total):
    """Shapes whose 128-query blocks overflow the 256 CUs while 160-query blocks fit in one round take
    five-wave query blocks: the ten-wave kernel that splits each block's key tiles into two halves
    (odd tile counts, ragged last tiles, chunk limits inside either half), or the five-wave kernel
    when a block holds a single key tile: against the oracle."""
    print("attention-five-wave", H, Lq, kv_base, chunk_q, kv_total, flush=True)
    assert -(-Lq // 128) * 2 * H > 256 and -(-Lq // 160) * 2 * H <= 256
    (out, out2), ref = _attn_case(gpu, "bf16", 2, H, 128, Lq, kv_base, chunk_q, kv_total, "w5_%d_%d_%d" % (H, Lq, kv_total),
                                  runs=2)
    assert np.all(np.isfinite(out))
    assert rel_l2(out, ref) <= 1e-2
    assert np.array_equal(out, out2)   # fixed order everywhere: a second run is bit-identical


@pytest.mark.timeout(600)
def test_op_attention_long_context_full_size_sampled(gpu):
    """Three-view long-context geometry at full size, as the step launches it (workspace given): 2
    branches x 40 heads of 128, a chunk of 1344 queries over 6 cached chunks + itself (9408 keys).
    The oracle computes 48 sampled query rows one by one."""
    br, H, d, Lq, kv_base = 2, 40, 128, 1344, 8064
    kv_total = kv_base + Lq
    print("attention-long-context-full", flush=True)
    k_rows = ((kv_total + 63) // 64) * 64 + 64
    v_stride = ((kv_total + 63) // 64) * 64
    q = draw((br, H, Lq, d), "lcq")
    k = draw((br, H, k_rows, d), "lck")
    v = draw((br, H, kv_total, d), "lcv")
    vt = np.zeros((br, H, d, v_stride), np.float32)
    vt[..., :kv_total] = np.swapaxes(v, -1, -2)
    Q, K, VT = (to_device(x, "bf16", gpu) for x in (q, k, vt))
    q = synth.round_bf16(q)
    k = synth.round_bf16(k)
    v = synth.round_bf16(v)
    Ot = torch.full((br * Lq, H * d), float("nan"), dtype=torch.bfloat16, device=gpu)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=gpu)
    wam.wam_op_attention(wam.WAM_BF16, Q, K, VT, Ot, br, H, d, Lq, k_rows, v_stride, kv_base, 0, kv_total, ws=ws)
    torch.cuda.synchronize()
    out = host(Ot).reshape(br, Lq, H, d)
    assert np.all(np.isfinite(out))
    u = synth.uniform01(3 * 48, synth.tensor_key(100, 0, "lc_samples"))
    picks = [(int(u[3 * i] * br), int(u[3 * i + 1] * H), int(u[3 * i + 2] * Lq)) for i in range(48)]
    picks += [(br - 1, H - 1, Lq - 1), (0, 0, 0)]
    got = np.stack([out[b, qi, h] for b, h, qi in picks])
    ref = np.stack([O.attention(q[b, h, qi:qi + 1].astype(np.float64), k[b, h, :kv_total].astype(np.float64),
                                v[b, h].astype(np.float64), None)[0] for b, h, qi in picks])
    assert rel_l2(got, ref) <= 1e-2


def test_op_attention_full_shape_bf16(gpu):
    """Config-3 self-attention geometry: 928 cached + 464 current keys, 40 heads of 128, 2 branches."""
    print("attention-full", flush=True)
    out, ref = _attn_case(gpu, "bf16", 2, 40, 128, 464, 928, 0, 1392, "full")
    assert rel_l2(out, ref) <= 1e-2


def _f32(x, gpu):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(gpu)


@pytest.mark.parametrize("M,N", [(1, 1024), (37, 5120), (928, 5120), (5, 8192), (3, 1028)])
@pytest.mark.parametrize("splits", [2, 3, 4])
@pytest.mark.parametrize("gate_idx,rms", [(5, False), (-1, False), (2, True)])
def test_op_split_finish(gpu, M, N, splits, gate_idx, rms):
    """The finishing row kernel of a split product against the oracle's residual update and
    modulated norm: h to fp32 rounding of its terms, y within a bf16 half-ulp; bit-identical rerun."""
    print("split-finish", M, N, splits, gate_idx, rms, flush=True)
    tag = "%d_%d_%d" % (M, N, splits)
    part = draw((splits, M, N), "part" + tag)
    h0 = draw((M, N), "h" + tag)
    bias = draw((N,), "fb" + tag, 0.1)
    e6 = draw((6, N), "e6" + tag, 0.1)
    mg = draw((6, N), "mg" + tag, 0.1)
    mn = draw((6, N), "mn" + tag, 0.1)
    shift_idx, scale_idx = (3, 4) if gate_idx == 2 else (0, 1)
    eps = 1e-6
    v = part.astype(np.float64).sum(axis=0) + bias
    gate = (e6[gate_idx].astype(np.float64) + mg[gate_idx]) if gate_idx >= 0 else np.ones(N)
    h_ref = h0 + gate * v
    y_ref = O.modulated_norm(h_ref, e6[shift_idx].astype(np.float64) + mn[shift_idx],
                             e6[scale_idx].astype(np.float64) + mn[scale_idx], eps, rms=rms)
    P, B, E, MG, MN = (_f32(x, gpu) for x in (part, bias, e6, mg, mn))
    outs = []
    for _ in range(2):
        H = _f32(h0, gpu)
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=gpu)
        wam.wam_op_split_finish(P, splits, M, N, B, H, E, MG if gate_idx >= 0 else None, gate_idx, MN, shift_idx,
                                scale_idx, Y, rms=rms, eps=eps)
        torch.cuda.synchronize()
        outs.append((H.cpu().numpy(), host(Y)))
    (h, y), (h2, y2) = outs
    assert np.array_equal(h, h2) and np.array_equal(y, y2)
    mag = np.abs(h0) + np.abs(gate) * (np.abs(part).sum(axis=0) + np.abs(bias))
    assert np.all(np.abs(h - h_ref) <= 4 * 2.0 ** -24 * mag)
    assert np.all(np.abs(y - y_ref) <= np.abs(y_ref) * 2.0 ** -8 + 1e-3)


@pytest.mark.parametrize("M,D", [(1, 64), (5, 100), (928, 5120), (33, 8192)])
@pytest.mark.parametrize("rms", [False, True])
def test_op_modulated_norm(gpu, M, D, rms):
    """The block's standalone adaLN kernel against the oracle's modulated norm (bf16 output)."""
    print("modulated-norm", M, D, rms, flush=True)
    tag = "%d_%d" % (M, D)
    x = draw((M, D), "nx" + tag, 2.0) + 0.5
    e6 = draw((6, D), "ne6" + tag, 0.1)
    mod = draw((6, D), "nmod" + tag, 0.1)
    y_ref = O.modulated_norm(x.astype(np.float64), e6[3].astype(np.float64) + mod[3],
                             e6[4].astype(np.float64) + mod[4], 1e-6, rms=rms)
    Y = torch.full((M, D), float("nan"), dtype=torch.bfloat16, device=gpu)
    wam.wam_op_modulated_norm(_f32(x, gpu), M, D, _f32(e6, gpu), _f32(mod, gpu), 3, 4, Y, rms=rms, eps=1e-6)
    torch.cuda.synchronize()
    assert np.all(np.abs(host(Y) - y_ref) <= np.abs(y_ref) * 2.0 ** -8 + 1e-3)


@pytest.mark.parametrize("br,rows,Lq,Lv,H,d,row0", [(2, 48, 24, 20, 4, 64, 16), (1, 8, 8, 8, 2, 128, 0),
                                                    (2, 464, 464, 440, 40, 128, 928)])
def test_op_qkv_cache(gpu, br, rows, Lq, Lv, H, d, row0):
    """q/k RMSNorm with gains, the rotary embedding of video rows and the scatter into head-major q and
    the caches, against the oracle's rms_norm and apply_rope; values copied bit for bit; cache rows
    outside [row0, row0 + rows) untouched; action rows ignore their (NaN) table entries."""
    print("qkv-cache", br, rows, Lq, Lv, H, d, row0, flush=True)
    D, eps, theta = H * d, 1e-6, 1e4
    cap = row0 + rows + 8
    tag = "%d_%d_%d_%d" % (br, rows, H, d)
    qkv = draw((br * rows, 3 * D), "qkv" + tag)
    gq = draw((D,), "gq" + tag, 0.1) + 1.0
    gk = draw((D,), "gk" + tag, 0.1) + 1.0
    rng = np.random.default_rng(rows + H)
    pos = np.stack([rng.integers(0, 24, rows), rng.integers(0, 11, rows), rng.integers(0, 20, rows)], axis=1)
    video = (np.arange(rows) % Lq) < Lv
    axis, freq = O.rope_frequencies(d, theta)
    ang = pos[:, axis].astype(np.float64) * freq[None, :]
    table = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)   # [rows][d/2][2]
    table[~video] = np.nan
    QKV = to_device(qkv, "bf16", gpu)
    Qo = torch.full((br, H, rows, d), float("nan"), dtype=torch.bfloat16, device=gpu)
    Kc = torch.full((br, H, cap, d), float("nan"), dtype=torch.bfloat16, device=gpu)
    Vc = torch.full((br, H, d, cap), float("nan"), dtype=torch.bfloat16, device=gpu)
    wam.wam_op_qkv_cache(QKV, br, rows, Lq, Lv, H, d, _f32(gq, gpu), _f32(gk, gpu), eps, _f32(table, gpu), Qo, Kc, Vc,
                         cap, row0)
    torch.cuda.synchronize()
    x = qkv.astype(np.float64).reshape(br, rows, 3, H, d)

    def expect(t, gain):
        out = np.empty((br, H, rows, d))
        for b in range(br):
            xn = O.rms_norm(x[b, :, t].reshape(rows, D), eps, gain.astype(np.float64)).reshape(rows, H, d)
            xn[video] = O.apply_rope(xn[video], pos[video], d, theta)
            out[b] = xn.transpose(1, 0, 2)
        return out

    q_ref, k_ref = expect(0, gq), expect(1, gk)
    q, k, v = host(Qo), host(Kc), host(Vc)
    assert np.all(np.abs(q - q_ref) <= np.abs(q_ref) * 2.0 ** -8 + 2e-3)
    assert np.all(np.abs(k[:, :, row0:row0 + rows] - k_ref) <= np.abs(k_ref) * 2.0 ** -8 + 2e-3)
    assert np.array_equal(v[:, :, :, row0:row0 + rows], x[:, :, 2].transpose(0, 2, 3, 1).astype(np.float32))
    assert np.isnan(k[:, :, :row0]).all() and np.isnan(k[:, :, row0 + rows:]).all()
    assert np.isnan(v[..., :row0]).all() and np.isnan(v[..., row0 + rows:]).all()
