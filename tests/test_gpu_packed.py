"""Fragment-packed projection weights through the C ABI (wam_pack_weight, wam_op_linear_packed,
wam_pack_block and the block's pk arena).

* The packed layout is checked element by element against its definition in the header (block
  (b, c) of 32 rows x 16 k at element offset (b K / 16 + c) 512, lane l holding row 32 b + l % 32 at
  k 16 c + 8 (l / 32) .. + 7): a pure permutation, so bit-exact.
* The packed product is checked against the float64 product of the same bf16 operands with the bound
  of the unpacked bf16 product (|gpu - ref| <= 2^-8 |ref| + 2^-8 1e-2: one bf16 rounding of an fp32
  sum of exact products), on shapes with ragged M and N (N a multiple of 32, not of the tile width).
* At the step's unsplit shapes it equals the unpacked product bit for bit: both kernels feed the same
  32x32x16 matrix instructions the same operands in the same k order (weight block first). The
  5120-wide products (over K = 5120 and K = 13824) take two K ranges packed (160 x 256 tiles)
  against three unpacked (192 x 320 tiles), so there they are held to the reference bound only.
* Stacks with packed weights (the unpacked copies of the six projections deleted) match the oracle
  within the bf16 stack bound 2e-2 relative L2.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import world_action_video_amd as wam
from synth.workloads import WORKLOADS, draw_named
from world_action_video_amd.device import DeviceCache, DeviceCtx, DeviceModel, to_device, workspace

pytestmark = pytest.mark.gpu


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def draw(shape, name, sigma=1.0):
    return synth.fill(shape, synth.tensor_key(101, 0, name), "normal", sigma=sigma)


def host(t):
    return t.float().cpu().numpy()


def packed(W, N, K, gpu):
    Wp = torch.empty(N * K, dtype=torch.bfloat16, device=gpu)
    wam.wam_pack_weight(W, K, N, K, Wp)
    return Wp


def split_ws(gpu, M, N):
    return torch.empty(4 * M * N * 4 + 256, dtype=torch.uint8, device=gpu)[:4 * M * N * 4]


@pytest.mark.parametrize("N,K,ldw", [(32, 64, 64), (96, 192, 200), (320, 512, 512)])
def test_pack_weight_layout(gpu, N, K, ldw):
    print("pack-layout", N, K, ldw, flush=True)
    w = draw((N, ldw), "pk%d_%d_%d" % (N, K, ldw))
    W = to_device(w, "bf16", gpu)
    Wp = torch.full((N * K,), float("nan"), dtype=torch.bfloat16, device=gpu)
    wam.wam_pack_weight(W, ldw, N, K, Wp)
    torch.cuda.synchronize()
    got = Wp.view(torch.int16).cpu().numpy()
    src = W.view(torch.int16).cpu().numpy()
    want = np.empty(N * K, np.int16)
    for b in range(N // 32):
        for c in range(K // 16):
            base = (b * (K // 16) + c) * 512
            for lane in range(64):
                r, k0 = 32 * b + lane % 32, 16 * c + 8 * (lane // 32)
                want[base + 8 * lane: base + 8 * lane + 8] = src[r, k0:k0 + 8]
    assert np.array_equal(got, want)


PACKED_CASES = [(1, 64, 64), (67, 224, 128), (300, 384, 512), (928, 1024, 256), (130, 96, 1024), (300, 544, 1024),
                (257, 800, 2048), (520, 16384, 320), (1024, 15360, 128)]


@pytest.mark.parametrize("M,N,K", PACKED_CASES)
@pytest.mark.parametrize("act", [0, 1, 2])
@pytest.mark.parametrize("split", [False, True])
def test_op_linear_packed_small(gpu, M, N, K, act, split):
    print("linear-packed", M, N, K, act, split, flush=True)
    a = draw((M, K), "a%d_%d_%d" % (M, N, K))
    w = draw((N, K), "w%d_%d_%d" % (M, N, K), 0.05)
    b = draw((N,), "b%d" % N, 0.1)
    ref = a.astype(np.float64) @ w.astype(np.float64).T + b
    if act == 1:
        ref = O.gelu_tanh(ref)
    elif act == 2:
        ref = O.silu(ref[:, 0::2]) * ref[:, 1::2]
    A, W = to_device(a, "bf16", gpu), to_device(w, "bf16", gpu)
    Wp = packed(W, N, K, gpu)
    del W
    B = torch.from_numpy(b).to(gpu)
    C = torch.full((M, N // 2 if act == 2 else N), float("nan"), dtype=torch.bfloat16, device=gpu)
    wam.wam_op_linear_packed(A, K, Wp, B, C, C.shape[1], M, N, K, act, ws=split_ws(gpu, M, N) if split else None)
    torch.cuda.synchronize()
    out = host(C)
    assert np.all(np.abs(out - ref) <= np.abs(ref) * 2.0 ** -8 + 2.0 ** -8 * 1e-2)


@pytest.mark.parametrize("M,N,K,split,act", [(928, 15360, 5120, False, 0), (928, 13824, 5120, False, 1),
                                             (928, 5120, 5120, True, 0), (928, 5120, 13824, True, 0),
                                             (2688, 5120, 5120, False, 0), (2688, 15360, 5120, False, 0)])
def test_op_linear_packed_full_size(gpu, M, N, K, split, act):
    """The step's projection shapes: equal, bit for bit, to the unpacked product where neither splits
    K (the 5120-wide split products take two K ranges packed, three unpacked), and within the reference bound on 4096
    sampled outputs; with a workspace the K ranges are summed in a fixed order, so a second run is
    identical too."""
    print("linear-packed-full", M, N, K, split, act, flush=True)
    a = draw((M, K), "fa%d_%d" % (M, K))
    w = draw((N, K), "fw%d_%d" % (N, K), 0.02)
    b = draw((N,), "fb%d" % N, 0.02)
    A, W = to_device(a, "bf16", gpu), to_device(w, "bf16", gpu)
    B = torch.from_numpy(b).to(gpu)
    ws = split_ws(gpu, M, N) if split else None
    C0 = torch.empty((M, N), dtype=torch.bfloat16, device=gpu)
    wam.wam_op_linear(wam.WAM_BF16, A, K, W, K, B, C0, N, M, N, K, act, ws=ws)
    Wp = packed(W, N, K, gpu)
    del W
    C = torch.empty_like(C0)
    wam.wam_op_linear_packed(A, K, Wp, B, C, N, M, N, K, act, ws=ws)
    C2 = torch.empty_like(C0)
    wam.wam_op_linear_packed(A, K, Wp, B, C2, N, M, N, K, act, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(C, C2)
    if not (split and N == 5120):   # two K ranges packed, three unpacked
        assert torch.equal(C, C0)
    out = host(C)
    rng = np.random.default_rng(11)
    rows = np.concatenate([rng.integers(0, M, 4000), [0, M - 1] * 48])
    cols = np.concatenate([rng.integers(0, N, 4000), [0, N - 1, N - 1, 0] * 24])
    a_bf = synth.round_bf16(a).astype(np.float64)
    w_bf = synth.round_bf16(w).astype(np.float64)
    ref = np.einsum("ik,ik->i", a_bf[rows], w_bf[cols]) + b[cols]
    if act == 1:
        ref = O.gelu_tanh(ref)
    assert np.all(np.abs(out[rows, cols] - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-3)


def _tiny_stack(gpu, variant, packed_w):
    w = WORKLOADS[1].with_(layers=2, variant=variant)
    m = O.load_model(w)
    txt = draw_named(w, -1, "txt")
    ctx = O.build_context(w, m.g, txt, None)
    ckv = [O.context_kv(w, lp, ctx) for lp in m.layers]
    x1v = [draw_named(w, -1, "x1_video_%d" % c) for c in range(2)]
    x1a = [draw_named(w, -1, "x1_action_%d" % c) for c in range(2)]
    epv, epa = draw_named(w, -1, "eps_video_1"), draw_named(w, -1, "eps_action_1")
    xv1, xa1 = O.interpolate(x1v[1], epv, 0.5), O.interpolate(x1a[1], epa, 0.5)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref = O.stack_forward(m, cache, ckv, xv1, xa1, [0.5], [0.5], 1, w.frames_per_chunk)

    dm = DeviceModel(w, "bf16", gpu, packed=packed_w)
    ws = workspace(dm.cfg, 2, gpu)
    dctx = DeviceCtx(w, "bf16", gpu)
    wam.wam_ctx_build(dm.cfg, dm.weights, to_device(txt, "bf16", gpu), None, dctx.c, ws)
    dc = DeviceCache(w, 3 * w.chunk_tokens, "bf16", gpu)
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(gpu)
    wam.wam_kv_append(dm.cfg, dm.weights, dc.c, dctx.c, f32(x1v[0]), f32(x1a[0]), 0, ws)
    br = dm.cfg.branches
    vv = torch.full((br, w.video_tokens, w.patch_dim), float("nan"), device=gpu)
    va = torch.full((br, w.action_tokens, w.action_dim), float("nan"), device=gpu)
    wam.wam_dit_stack_fwd(dm.cfg, dm.weights, dc.c, dctx.c, 1, f32(xv1), f32(xa1), [0.5], [0.5], w.frames_per_chunk,
                          vv, va, ws)
    torch.cuda.synchronize()
    return ref, (vv.cpu().numpy(), va.cpu().numpy())


@pytest.mark.parametrize("variant", [0, synth.workloads.VARIANT_SWIGLU | synth.workloads.VARIANT_RMS_NORM])
def test_stack_tiny_packed_matches_oracle(gpu, variant):
    """Two layers at width 256 (products far below one round of tiles: ragged M, split K) with only
    the packed copies of the six projections on the device."""
    print("stack-tiny-packed", variant, flush=True)
    (ref_v, ref_a), (gv, ga) = _tiny_stack(gpu, variant, True)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert np.all(np.isfinite(gv)) and np.all(np.isfinite(ga))
    assert ev <= 2e-2 and ea <= 2e-2
