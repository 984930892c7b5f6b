"""Stack-level parity of the HIP path (through the C ABI) against the CPU oracle, and the GPU-side
invariants the pages fix. Tolerances (relative L2 per output tensor, video and action apart):
2e-2 in bf16 and 1e-4 in the fp32 debug mode.
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

TOL = {"bf16": 2e-2, "f32": 1e-4}


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


class Rig:
    """GPU model + condition KV for one workload and dtype, plus the host copies of its inputs."""

    def __init__(self, w, dtype, device):
        self.w, self.dtype, self.dev = w, dtype, device
        self.m = DeviceModel(w, dtype, device)
        self.ws = workspace(self.m.cfg, 2, device)
        self.txt = draw_named(w, -1, "txt")
        self.img = draw_named(w, -1, "img") if w.ctx_img_len else None
        self.ctx = DeviceCtx(w, dtype, device)
        self.state = draw_named(w, -1, "state_0") if w.ctx_state_len else None
        wam.wam_ctx_build(self.m.cfg, self.m.weights, to_device(self.txt, dtype, device),
                          to_device(self.img, dtype, device) if self.img is not None else None, self.ctx.c, self.ws,
                          state=to_device(self.state, dtype, device) if self.state is not None else None)

    def cache(self, chunks=3):
        return DeviceCache(self.w, chunks * self.w.chunk_tokens, self.dtype, self.dev)

    def f32(self, x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(self.dev)

    def append(self, cache, xv, xa, start):
        wam.wam_kv_append(self.m.cfg, self.m.weights, cache.c, self.ctx.c, self.f32(xv), self.f32(xa), start, self.ws)

    def step(self, cache, n, xv, xa, tv, ta, start):
        w = self.w
        br = self.m.cfg.branches
        vv = torch.full((br, n * w.video_tokens, w.patch_dim), float("nan"), device=self.dev)
        va = torch.full((br, n * w.action_tokens, w.action_dim), float("nan"), device=self.dev)
        wam.wam_dit_stack_fwd(self.m.cfg, self.m.weights, cache.c, self.ctx.c, n, self.f32(xv), self.f32(xa), tv, ta,
                              start, vv, va, self.ws)
        torch.cuda.synchronize()
        return vv.cpu().numpy(), va.cpu().numpy()


def tiny_inputs(w):
    x1v = [draw_named(w, -1, "x1_video_%d" % c) for c in range(3)]
    x1a = [draw_named(w, -1, "x1_action_%d" % c) for c in range(3)]
    epv = [draw_named(w, -1, "eps_video_%d" % c) for c in range(3)]
    epa = [draw_named(w, -1, "eps_action_%d" % c) for c in range(3)]
    return x1v, x1a, epv, epa


@pytest.fixture(scope="module")
def tiny_oracle():
    w = WORKLOADS[1].with_(layers=2)
    m = O.load_model(w)
    txt = draw_named(w, -1, "txt")
    ctx = O.build_context(w, m.g, txt, None)
    ckv = [O.context_kv(w, lp, ctx) for lp in m.layers]
    return w, m, ckv


@pytest.mark.parametrize("P,A", [(32, 8), (16, 40), (48, 64)])
def test_stack_tiny_head_widths_bf16(gpu, P, A):
    """Patch and action widths that give the output heads one or two 32-column blocks each (the
    benchmarked shapes have 64 and 8): the bf16 step of a one-layer tiny model against the oracle."""
    w = WORKLOADS[1].with_(layers=1, patch_dim=P, action_dim=A)
    print("stack-tiny-heads", P, A, flush=True)
    m = O.load_model(w)
    txt = draw_named(w, -1, "txt")
    ckv = [O.context_kv(w, lp, O.build_context(w, m.g, txt, None)) for lp in m.layers]
    x1v, x1a, epv, epa = tiny_inputs(w)
    xv1 = O.interpolate(x1v[1], epv[1], 0.5)
    xa1 = O.interpolate(x1a[1], epa[1], 0.5)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, xv1, xa1, [0.5], [0.5], 1, w.frames_per_chunk)
    rig = Rig(w, "bf16", gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    gv, ga = rig.step(dc, 1, xv1, xa1, [0.5], [0.5], w.frames_per_chunk)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert gv.shape[-1] == P and ga.shape[-1] == A
    assert np.all(np.isfinite(gv)) and np.all(np.isfinite(ga))
    assert ev <= TOL["bf16"] and ea <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stack_tiny_matches_oracle(gpu, tiny_oracle, dtype):
    w, m, ckv = tiny_oracle
    print("stack-tiny", dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    xv1 = O.interpolate(x1v[1], epv[1], 0.5)
    xa1 = O.interpolate(x1a[1], epa[1], 0.5)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, xv1, xa1, [0.5], [0.5], 1, w.frames_per_chunk)

    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    assert dc.length == w.chunk_tokens
    gv, ga = rig.step(dc, 1, xv1, xa1, [0.5], [0.5], w.frames_per_chunk)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert np.all(np.isfinite(gv)) and np.all(np.isfinite(ga))
    assert ev <= TOL[dtype] and ea <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_three_camera_grid(gpu, tiny_oracle, dtype):
    """The three-camera 352 x 640 input of the single-GPU inference docs: 22 x 40 patches per frame
    (880 tokens), 1784 tokens per chunk with the actions, rotary rows and columns up to 21 and 39,
    one cached chunk, on the tiny width."""
    w0, m0, ckv = tiny_oracle
    w = w0.with_(grid_h=22, grid_w=40)
    m = O.Model(w, m0.g, m0.layers)
    print("three-camera grid", dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    xv1 = O.interpolate(x1v[1], epv[1], 0.5)
    xa1 = O.interpolate(x1a[1], epa[1], 0.5)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, xv1, xa1, [0.5], [0.5], 1, w.frames_per_chunk)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache(2)
    rig.append(dc, x1v[0], x1a[0], 0)
    gv, ga = rig.step(dc, 1, xv1, xa1, [0.5], [0.5], w.frames_per_chunk)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_frame_causal_variant(gpu, tiny_oracle, dtype):
    """Frame-causal mask inside the chunk (architecture page's causal-mask drawing): against the
    oracle; on the GPU, the second frame and the action tokens cannot reach the first frame's
    outputs, bit for bit; incremental equals full-sequence."""
    w0, m0, ckv = tiny_oracle
    w = w0.with_(variant=synth.workloads.VARIANT_FRAME_CAUSAL)
    m = O.Model(w, m0.g, m0.layers)
    hw, Lv, La, Fc = w.grid_h * w.grid_w, w.video_tokens, w.action_tokens, w.frames_per_chunk
    print("frame-causal", dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.4], [0.4], 1, Fc)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    gv, ga = rig.step(dc, 1, epv[1], epa[1], [0.4], [0.4], Fc)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]
    xv2 = epv[1].copy()
    xv2[hw:] = xv2[hw:] * 3 - 1
    pv, pa = rig.step(dc, 1, xv2, epa[1], [0.4], [0.4], Fc)
    assert np.array_equal(pv[:, :hw], gv[:, :hw]) and not np.array_equal(pa, ga)
    qv, qa = rig.step(dc, 1, epv[1], -epa[1], [0.4], [0.4], Fc)
    assert np.array_equal(qv, gv) and not np.array_equal(qa, ga)
    fv, fa = rig.step(rig.cache(), 2, np.concatenate([x1v[0], epv[1]]), np.concatenate([x1a[0], epa[1]]),
                      [1.0, 0.4], [1.0, 0.4], 0)
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert rel_l2(fv[:, Lv:], gv) <= tol and rel_l2(fa[:, La:], ga) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [synth.workloads.VARIANT_RMS_NORM,
                                     synth.workloads.VARIANT_RMS_NORM | synth.workloads.VARIANT_FRAME_CAUSAL,
                                     synth.workloads.VARIANT_SWIGLU,
                                     synth.workloads.VARIANT_SWIGLU | synth.workloads.VARIANT_RMS_NORM
                                     | synth.workloads.VARIANT_FRAME_CAUSAL])
def test_variant_stack_matches_oracle(gpu, tiny_oracle, dtype, variant):
    """Architectural variants (RMSNorm block and head norms, SwiGLU feed-forward, combined with the
    frame-causal mask): one cached chunk and a step, against the oracle with the same variant."""
    w0, m0, ckv = tiny_oracle
    w = w0.with_(variant=variant)
    # SwiGLU draws a wider first feed-forward matrix; every other tensor is drawn identically
    m = O.load_model(w) if variant & synth.workloads.VARIANT_SWIGLU else O.Model(w, m0.g, m0.layers)
    print("variant", variant, dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.35], [0.55], 1, w.frames_per_chunk)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    gv, ga = rig.step(dc, 1, epv[1], epa[1], [0.35], [0.55], w.frames_per_chunk)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]


# MXFP8 projections against the oracle taking the same quantised projections. Both sides quantise
# the bf16 rows of the projection inputs (the oracle rounds its fp32 activations to bf16 first, as
# the library stores them), so what remains is the bf16 path's own difference, whose bar is 2e-2; at
# this width it flips few fp8 codes (measured 2.3e-3 / 6.2e-3 at most, video / action).
MX_TOL = 2e-2


@pytest.mark.parametrize("precision", [synth.workloads.PRECISION_MXFP8, synth.workloads.PRECISION_MXFP4W])
@pytest.mark.parametrize("variant", [0, synth.workloads.VARIANT_SWIGLU | synth.workloads.VARIANT_RMS_NORM])
def test_mxfp8_stack_matches_oracle(gpu, tiny_oracle, variant, precision):
    """One cached chunk and a step with the six block projections in MXFP8 (or MXFP4 weights with
    MXFP8 activations), against the oracle with the same quantised projections; the distance to the
    unquantised model is printed (quality). The weights are quantised identically on both sides (the
    quantisers are bit-exact), so the bound is the MXFP8 one."""
    w0, m0, ckv = tiny_oracle
    w = w0.with_(variant=variant, precision=precision)
    m = O.load_model(w) if variant & synth.workloads.VARIANT_SWIGLU else O.Model(w, m0.g, m0.layers)
    print("low-precision stack, precision", precision, "variant", variant, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.35], [0.55], 1, w.frames_per_chunk)
    wn = w.with_(precision=0)
    mn = O.Model(wn, m.g, m.layers)
    cn = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(mn, cn, ckv, x1v[0], x1a[0], 0)
    nat_v, nat_a = O.stack_forward(mn, cn, ckv, epv[1], epa[1], [0.35], [0.55], 1, w.frames_per_chunk)
    rig = Rig(w, "bf16", gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    gv, ga = rig.step(dc, 1, epv[1], epa[1], [0.35], [0.55], w.frames_per_chunk)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 to the MXFP8 oracle: video %.3e action %.3e; oracle MXFP8 to unquantised: video %.3e "
          "action %.3e" % (ev, ea, rel_l2(ref_v, nat_v), rel_l2(ref_a, nat_a)), flush=True)
    assert ev <= MX_TOL and ea <= MX_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [synth.workloads.VARIANT_IMG_XATTN,
                                     synth.workloads.VARIANT_IMG_XATTN | synth.workloads.VARIANT_FRAME_CAUSAL])
def test_separate_image_attention(gpu, dtype, variant):
    """Image condition tokens with their own key / value projections and softmax (16 image tokens after
    32 text tokens): condition build, one cached chunk and a step, against the oracle."""
    w = WORKLOADS[1].with_(layers=2, ctx_img_len=16, variant=variant)
    m = O.load_model(w)
    ctx = O.build_context(w, m.g, draw_named(w, -1, "txt"), draw_named(w, -1, "img"))
    ckv = [O.context_kv(w, lp, ctx) for lp in m.layers]
    x1v, x1a, epv, epa = tiny_inputs(w)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.3], [0.6], 1, w.frames_per_chunk)
    print("image cross-attention", variant, dtype, flush=True)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    gv, ga = rig.step(dc, 1, epv[1], epa[1], [0.3], [0.6], w.frames_per_chunk)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]


def test_qkv_timer(gpu, tiny_oracle):
    """The QKV measurement hook: one sample per pass through the chosen layer (none from the key/value
    only product of an append's last layer, none past max_samples), positive durations, and the
    read restarts the count; disabled, nothing is recorded."""
    w0, _, _ = tiny_oracle
    w = w0.with_(layers=2)
    x1v, x1a, epv, epa = tiny_inputs(w)
    rig = Rig(w, "bf16", gpu)
    dc = rig.cache()
    wam.wam_qkv_timer_config(1, 2)
    try:
        rig.append(dc, x1v[0], x1a[0], 0)          # layer 1 is the last: keys/values only
        assert wam.wam_qkv_timer_read() == []
        for _ in range(3):
            rig.step(dc, 1, epv[1], epa[1], [0.5], [0.5], w.frames_per_chunk)
        ms = wam.wam_qkv_timer_read()
        assert len(ms) == 2 and all(0.0 < t < 100.0 for t in ms)
        assert wam.wam_qkv_timer_read() == []
    finally:
        wam.wam_qkv_timer_config(-1)
    rig.step(dc, 1, epv[1], epa[1], [0.5], [0.5], w.frames_per_chunk)
    assert wam.wam_qkv_timer_read() == []


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_state", [1, 3, 6])
def test_state_rows(gpu, tiny_oracle, dtype, n_state):
    """Proprioceptive state rows in the condition sequence: built with the first observed state, a
    step against the oracle; then the state rows alone updated to a new observation
    (wam_ctx_set_state) and the step again, against the oracle rebuilt with the new state. Up to
    four rows take the row-parallel product, more the tiled GEMM."""
    _, _, _ = tiny_oracle
    w = WORKLOADS[1].with_(layers=2, ctx_state_len=n_state)
    m = O.load_model(w)
    txt = draw_named(w, -1, "txt")
    x1v, x1a, epv, epa = tiny_inputs(w)
    rig = Rig(w, dtype, gpu)
    for c in (0, 1):
        st = draw_named(w, -1, "state_%d" % c)
        if c == 1:
            wam.wam_ctx_set_state(rig.m.cfg, rig.m.weights, to_device(st, dtype, gpu), rig.ctx.c, rig.ws)
        ckv = [O.context_kv(w, lp, O.build_context(w, m.g, txt, None, st)) for lp in m.layers]
        cache = O.KVCache.empty(w.layers, w.branches, w.dim)
        O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
        ref_v, ref_a = O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.45], [0.45], 1, w.frames_per_chunk)
        dc = rig.cache()
        rig.append(dc, x1v[0], x1a[0], 0)
        gv, ga = rig.step(dc, 1, epv[1], epa[1], [0.45], [0.45], w.frames_per_chunk)
        ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
        print("state %d x%d %s: rel-L2 video %.3e action %.3e" % (c, n_state, dtype, ev, ea), flush=True)
        assert ev <= TOL[dtype] and ea <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_embodiment_routing(gpu, tiny_oracle, dtype):
    """Three embodiments in one model: each request routed by id runs that embodiment's action encoder
    and decoder (append and step), against the oracle with the same routing; the default weights
    stay embodiment 0's."""
    w0, m0, ckv = tiny_oracle
    w = w0.with_(embodiments=3)
    m = O.load_model(w)
    x1v, x1a, epv, epa = tiny_inputs(w)
    rig = Rig(w, dtype, gpu)
    outs = []
    for e in (2, 0, 1):
        me = O.Model(w, O.embodiment_params(m.g, e), m.layers)
        cache = O.KVCache.empty(w.layers, w.branches, w.dim)
        O.kv_append(me, cache, ckv, x1v[0], x1a[0], 0)
        ref_v, ref_a = O.stack_forward(me, cache, ckv, epv[1], epa[1], [0.4], [0.4], 1, w.frames_per_chunk)
        rig.m.weights_routed = rig.m.for_embodiment(e)
        default = rig.m.weights
        rig.m.weights = rig.m.weights_routed
        try:
            dc = rig.cache()
            rig.append(dc, x1v[0], x1a[0], 0)
            gv, ga = rig.step(dc, 1, epv[1], epa[1], [0.4], [0.4], w.frames_per_chunk)
        finally:
            rig.m.weights = default
        ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
        print("embodiment %d: rel-L2 video %.3e action %.3e" % (e, ev, ea), flush=True)
        assert ev <= TOL[dtype] and ea <= TOL[dtype]
        outs.append(ga)
    assert not np.allclose(outs[0], outs[1]) and not np.allclose(outs[1], outs[2])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decoupled_timesteps_and_frames(gpu, tiny_oracle, dtype):
    """Different video/action timesteps and a non-zero window offset, two cached chunks."""
    w, m, ckv = tiny_oracle
    print("stack-tiny-decoupled", dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    Fc = w.frames_per_chunk
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 3)
    O.kv_append(m, cache, ckv, x1v[1], x1a[1], 3 + Fc)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, epv[2], epa[2], [0.1], [0.8], 1, 3 + 2 * Fc)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 3)
    rig.append(dc, x1v[1], x1a[1], 3 + Fc)
    gv, ga = rig.step(dc, 1, epv[2], epa[2], [0.1], [0.8], 3 + 2 * Fc)
    assert rel_l2(gv, ref_v) <= TOL[dtype] and rel_l2(ga, ref_a) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_incremental_equals_full_sequence_gpu(gpu, tiny_oracle, dtype):
    w, _, _ = tiny_oracle
    print("inc-vs-full", dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    Lv, La = w.video_tokens, w.action_tokens
    xv1 = O.interpolate(x1v[1], epv[1], 0.25)
    xa1 = O.interpolate(x1a[1], epa[1], 0.25)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    iv, ia = rig.step(dc, 1, xv1, xa1, [0.25], [0.25], w.frames_per_chunk)
    fc = rig.cache()
    fv, fa = rig.step(fc, 2, np.concatenate([x1v[0], xv1]), np.concatenate([x1a[0], xa1]), [1.0, 0.25], [1.0, 0.25], 0)
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert rel_l2(fv[:, Lv:], iv) <= tol and rel_l2(fa[:, La:], ia) <= tol
    print("bitwise equal:", np.array_equal(fv[:, Lv:], iv), flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_future_perturbation_bit_identical_gpu(gpu, tiny_oracle, dtype):
    w, _, _ = tiny_oracle
    print("perturb", dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    Lv, La = w.video_tokens, w.action_tokens
    rig = Rig(w, dtype, gpu)
    a = rig.step(rig.cache(), 2, np.concatenate([x1v[0], epv[1]]), np.concatenate([x1a[0], epa[1]]), [1, .2], [1, .2], 0)
    b = rig.step(rig.cache(), 2, np.concatenate([x1v[0], epv[1] * 7 + 3]), np.concatenate([x1a[0], -epa[1]]),
                 [1, .9], [1, .6], 0)
    assert np.array_equal(a[0][:, :Lv], b[0][:, :Lv]) and np.array_equal(a[1][:, :La], b[1][:, :La])
    assert not np.array_equal(a[0][:, Lv:], b[0][:, Lv:])


def test_run_to_run_bitwise_determinism(gpu, tiny_oracle):
    w, _, _ = tiny_oracle
    x1v, x1a, epv, epa = tiny_inputs(w)
    rig = Rig(w, "bf16", gpu)
    outs = []
    for _ in range(2):
        dc = rig.cache()
        rig.append(dc, x1v[0], x1a[0], 0)
        outs.append(rig.step(dc, 1, epv[1], epa[1], [0.3], [0.3], w.frames_per_chunk))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_reset_then_reappend_equals_fresh_cache(gpu, tiny_oracle, dtype):
    """Continuous requests (single-GPU docs: at a window boundary the old KV is released and the frame
    position restarts): after two committed chunks and wam_kv_reset, appending a chunk at frame 0 and
    stepping gives bit for bit what a fresh cache gives; the stale rows left past the new length never
    reach the output."""
    w, _, _ = tiny_oracle
    Fc = w.frames_per_chunk
    print("kv-reset", dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    rig = Rig(w, dtype, gpu)
    fresh = rig.cache()
    rig.append(fresh, x1v[2], x1a[2], 0)
    ref = rig.step(fresh, 1, epv[1], epa[1], [0.3], [0.3], Fc)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    rig.append(dc, x1v[1], x1a[1], Fc)
    rig.step(dc, 1, epv[2], epa[2], [0.6], [0.6], 2 * Fc)   # also writes scratch rows past the length
    wam.wam_kv_reset(dc.c)
    assert dc.length == 0
    rig.append(dc, x1v[2], x1a[2], 0)
    assert dc.length == w.chunk_tokens
    got = rig.step(dc, 1, epv[1], epa[1], [0.3], [0.3], Fc)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cfg_batch_equals_two_single_branch_calls(gpu, tiny_oracle, dtype):
    """CFG as batch 2 computes each branch exactly as a one-branch call would. Every row of the
    step is independent of the other branch, so the fp32 path (one kernel configuration for any row
    count) must agree bit for bit. In bf16 the row count picks the product kernel and may split a
    product over K (different fp32 summation order, then bf16 rounding), so there the two agree to
    within a few bf16 roundings: relative L2 <= 5e-3, a quarter of the oracle bar."""
    w, _, _ = tiny_oracle
    x1v, x1a, epv, epa = tiny_inputs(w)
    rig2 = Rig(w, dtype, gpu)
    dc = rig2.cache()
    rig2.append(dc, x1v[0], x1a[0], 0)
    both = rig2.step(dc, 1, epv[1], epa[1], [0.3], [0.3], w.frames_per_chunk)
    w1 = w.with_(branches=1)
    for b in range(2):
        m1 = DeviceModel(w1, dtype, gpu)
        ws = workspace(m1.cfg, 1, gpu)
        ctx1 = DeviceCtx(w1, dtype, gpu)
        wam.wam_ctx_build(m1.cfg, m1.weights, to_device(rig2.txt[b:b + 1], dtype, gpu), None, ctx1.c, ws)
        c1 = DeviceCache(w1, 2 * w.chunk_tokens, dtype, gpu)
        f32 = rig2.f32
        wam.wam_kv_append(m1.cfg, m1.weights, c1.c, ctx1.c, f32(x1v[0]), f32(x1a[0]), 0, ws)
        vv = torch.empty((1, w.video_tokens, w.patch_dim), device=gpu)
        va = torch.empty((1, w.action_tokens, w.action_dim), device=gpu)
        wam.wam_dit_stack_fwd(m1.cfg, m1.weights, c1.c, ctx1.c, 1, f32(epv[1]), f32(epa[1]), [0.3], [0.3],
                              w.frames_per_chunk, vv, va, ws)
        torch.cuda.synchronize()
        gv, ga = vv.cpu().numpy()[0], va.cpu().numpy()[0]
        if dtype == "f32":
            assert np.array_equal(gv, both[0][b]) and np.array_equal(ga, both[1][b])
        else:
            ev, ea = rel_l2(gv, both[0][b]), rel_l2(ga, both[1][b])
            print("branch", b, "rel-L2 video %.2e action %.2e" % (ev, ea), flush=True)
            assert ev <= 5e-3 and ea <= 5e-3


_DENOISE_REF = {}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tau,max_reuse,calls_expected", [(1.5, -1, 16), (-1.5, -1, 2), (-1.5, 1, 9)])
def test_denoise_chunk_matches_oracle(gpu, tiny_oracle, dtype, tau, max_reuse, calls_expected):
    """The library's 16-step Euler loop with velocity reuse (wam_denoise_chunk) against the oracle's
    loop on the same DiT: same call count and reuse pattern (the thresholds are far from any cosine,
    so the decisions cannot differ), final latents within the stack tolerance."""
    w, m, ckv = tiny_oracle
    x1v, x1a, epv, epa = tiny_inputs(w)
    grid = [k / 16 for k in range(17)]
    key = (tau, max_reuse)
    if key not in _DENOISE_REF:
        cache = O.KVCache.empty(w.layers, w.branches, w.dim)
        O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)

        def dit(xv, xa, t):
            vb, ab = O.stack_forward(m, cache, ckv, xv, xa, [t], [t], 1, w.frames_per_chunk)
            return O.cfg_combine(vb, w.guidance), O.cfg_combine(ab, w.guidance)
        _DENOISE_REF[key] = O.denoise_chunk(dit, epv[1], epa[1], grid, tau, None if max_reuse < 0 else max_reuse)
    ref_v, ref_a, n_ref, flags_ref = _DENOISE_REF[key]
    print("denoise", dtype, tau, max_reuse, flush=True)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    xv, xa = rig.f32(epv[1]), rig.f32(epa[1])
    br = rig.m.cfg.branches
    vv = torch.empty((br, w.video_tokens, w.patch_dim), device=gpu)
    va = torch.empty((br, w.action_tokens, w.action_dim), device=gpu)
    gv = torch.empty(w.video_tokens * w.patch_dim, device=gpu)
    ga = torch.empty(w.action_tokens * w.action_dim, device=gpu)
    cosp = torch.empty(3, device=gpu)
    calls, flags = wam.wam_denoise_chunk(rig.m.cfg, rig.m.weights, dc.c, rig.ctx.c, xv, xa, grid, w.guidance, tau, vv, va,
                                         gv, ga, cosp, rig.ws, start_frame=w.frames_per_chunk,
                                         max_consecutive_reuse=max_reuse)
    torch.cuda.synchronize()
    assert calls == n_ref == calls_expected
    assert flags == list(flags_ref)
    ev, ea = rel_l2(xv.cpu().numpy(), ref_v), rel_l2(xa.cpu().numpy(), ref_a)
    print("rel-L2 video %.2e action %.2e" % (ev, ea), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]


_UNIPC_REF = {}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("order,corrector,tau,max_reuse", [(2, True, 1.5, -1), (3, True, 1.5, -1),
                                                           (2, False, 1.5, -1), (1, True, 1.5, -1),
                                                           (2, True, -1.5, 1)])
def test_denoise_chunk_unipc_matches_oracle(gpu, tiny_oracle, dtype, order, corrector, tau, max_reuse):
    """The library's 16-step UniPC loop (wam_denoise_chunk_unipc) against the oracle's UniPC loop on
    the same DiT: same calls and reuse pattern, final latents within the stack tolerance."""
    w, m, ckv = tiny_oracle
    x1v, x1a, epv, epa = tiny_inputs(w)
    grid = [k / 16 for k in range(17)]
    key = (order, corrector, tau, max_reuse)
    if key not in _UNIPC_REF:
        cache = O.KVCache.empty(w.layers, w.branches, w.dim)
        O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)

        def dit(xv, xa, t):
            vb, ab = O.stack_forward(m, cache, ckv, xv, xa, [t], [t], 1, w.frames_per_chunk)
            return O.cfg_combine(vb, w.guidance), O.cfg_combine(ab, w.guidance)
        _UNIPC_REF[key] = O.denoise_chunk_unipc(dit, epv[1], epa[1], grid, tau, None if max_reuse < 0 else max_reuse,
                                                order=order, corrector=corrector)
    ref_v, ref_a, n_ref, flags_ref = _UNIPC_REF[key]
    print("unipc", dtype, key, flush=True)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    xv, xa = rig.f32(epv[1]), rig.f32(epa[1])
    br = rig.m.cfg.branches
    n = w.video_tokens * w.patch_dim + w.action_tokens * w.action_dim
    vv = torch.empty((br, w.video_tokens, w.patch_dim), device=gpu)
    va = torch.empty((br, w.action_tokens, w.action_dim), device=gpu)
    gv = torch.empty(w.video_tokens * w.patch_dim, device=gpu)
    ga = torch.empty(w.action_tokens * w.action_dim, device=gpu)
    cosp = torch.empty(3, device=gpu)
    state = torch.full((5 * n,), float("nan"), device=gpu)   # contents on entry must not matter
    calls, flags = wam.wam_denoise_chunk_unipc(rig.m.cfg, rig.m.weights, dc.c, rig.ctx.c, xv, xa, grid, w.guidance, tau,
                                               vv, va, gv, ga, cosp, state, rig.ws, order=order, corrector=corrector,
                                               start_frame=w.frames_per_chunk, max_consecutive_reuse=max_reuse)
    torch.cuda.synchronize()
    assert calls == n_ref
    assert flags == list(flags_ref)
    ev, ea = rel_l2(xv.cpu().numpy(), ref_v), rel_l2(xa.cpu().numpy(), ref_a)
    print("rel-L2 video %.2e action %.2e" % (ev, ea), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]


@pytest.mark.parametrize("nv,na", [(28160, 192), (28161, 193), (9_000_000, 4096)])
def test_flow_step_matches_oracle(gpu, nv, na):
    """The step's latent sizes (440 x 64 video and 24 x 8 action elements per branch; float4 path), odd
    sizes (scalar path) and a large latent whose grid reaches the 512-workgroup limit."""
    rng = synth.tensor_key(101, 0, "flow")
    v = synth.fill((2, nv + na), rng, "normal", 1.0)
    xv = synth.fill((nv,), rng + 1, "normal", 1.0)
    xa = synth.fill((na,), rng + 2, "normal", 1.0)
    prev = synth.fill((nv,), rng + 3, "normal", 1.0)
    vv, va = np.ascontiguousarray(v[:, :nv]), np.ascontiguousarray(v[:, nv:])
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(gpu)  # noqa: E731
    Xv, Xa, Prev = d(xv), d(xa), d(prev)
    Gv, Ga = torch.empty(nv, device=gpu), torch.empty(na, device=gpu)
    cos = torch.empty(3, device=gpu)
    ws = torch.empty(32768, dtype=torch.uint8, device=gpu)
    wam.wam_flow_step(Xv, Xa, d(vv), d(va), 2, 5.0, nv, na, 1 / 16, 0.25, Gv, Ga, Prev, cos, ws)
    torch.cuda.synchronize()
    gv = O.cfg_combine(vv, 5.0)
    ga = O.cfg_combine(va, 5.0)
    np.testing.assert_allclose(Gv.cpu().numpy(), gv, rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(Ga.cpu().numpy(), ga, rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(Xv.cpu().numpy(), O.euler_update(xv, gv, 0.0, 1 / 16), rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(Xa.cpu().numpy(), O.euler_update(xa, ga, 0.0, 0.25), rtol=2e-6, atol=2e-6)
    c = cos.cpu().numpy().astype(np.float64)
    g64 = gv.astype(np.float64)
    p64 = prev.astype(np.float64)
    np.testing.assert_allclose(c, [g64 @ p64, g64 @ g64, p64 @ p64], rtol=1e-4, atol=1e-2)
    assert abs(c[0] / np.sqrt(c[1] * c[2]) - O.cosine_fp64(gv, prev)) < 1e-5
    # guidance 1 returns the conditional branch exactly; one branch = plain Euler
    Xv2 = d(xv)
    Gv2 = torch.empty(nv, device=gpu)
    wam.wam_flow_step(Xv2, Xa, d(vv), d(va), 2, 1.0, nv, na, 0.5, 0.5, Gv2, None, None, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(Gv2.cpu().numpy(), vv[0])


@pytest.mark.parametrize("nv,na", [(28160, 192), (1_000_000, 4096)])
def test_flow_step_single_branch_and_cosine_only(gpu, nv, na):
    """The float4 path's other cases: one branch (the velocity is the guided velocity, no guidance
    arithmetic) with the cosine but no stored video velocity, and two branches with the cosine and
    neither velocity stored; both against the oracle's Euler update and fp64 cosine."""
    rng = synth.tensor_key(101, 2, "flow-cases")
    v = synth.fill((2, nv + na), rng, "normal", 1.0)
    xv = synth.fill((nv,), rng + 1, "normal", 1.0)
    xa = synth.fill((na,), rng + 2, "normal", 1.0)
    prev = synth.fill((nv,), rng + 3, "normal", 1.0)
    vv, va = np.ascontiguousarray(v[:, :nv]), np.ascontiguousarray(v[:, nv:])
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(gpu)  # noqa: E731
    ws = torch.empty(32768, dtype=torch.uint8, device=gpu)
    for br in (1, 2):
        print("flow-cases", nv, na, br, flush=True)
        Xv, Xa, cos = d(xv), d(xa), torch.empty(3, device=gpu)
        Ga = torch.empty(na, device=gpu) if br == 1 else None
        wam.wam_flow_step(Xv, Xa, d(vv[:br]), d(va[:br]), br, 5.0, nv, na, 1 / 16, 0.25, None, Ga, d(prev), cos, ws)
        torch.cuda.synchronize()
        gv = vv[0] if br == 1 else O.cfg_combine(vv, 5.0)
        ga = va[0] if br == 1 else O.cfg_combine(va, 5.0)
        if br == 1:
            assert np.array_equal(Ga.cpu().numpy(), va[0])
        np.testing.assert_allclose(Xv.cpu().numpy(), O.euler_update(xv, gv, 0.0, 1 / 16), rtol=2e-6, atol=2e-6)
        np.testing.assert_allclose(Xa.cpu().numpy(), O.euler_update(xa, ga, 0.0, 0.25), rtol=2e-6, atol=2e-6)
        c = cos.cpu().numpy().astype(np.float64)
        assert abs(c[0] / np.sqrt(c[1] * c[2]) - O.cosine_fp64(gv, prev)) < 1e-5


@pytest.mark.parametrize("nv,na", [(0, 192), (28160, 0), (5, 3)])
def test_flow_step_one_group_or_tiny(gpu, nv, na):
    """Degenerate sizes: no video part, no action part, and fewer elements than one vector (the scalar
    path): the Euler update of what is there, nothing else touched."""
    rng = synth.tensor_key(101, 1, "flow-edge")
    v = synth.fill((2, nv + na), rng, "normal", 1.0)
    xv = synth.fill((max(nv, 1),), rng + 1, "normal", 1.0)
    xa = synth.fill((max(na, 1),), rng + 2, "normal", 1.0)
    vv, va = np.ascontiguousarray(v[:, :nv]), np.ascontiguousarray(v[:, nv:])
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(gpu)  # noqa: E731
    Xv, Xa = d(xv), d(xa)
    ws = torch.empty(4096, dtype=torch.uint8, device=gpu)
    wam.wam_flow_step(Xv, Xa, d(vv) if nv else None, d(va) if na else None, 2, 5.0, nv, na, 0.25, 0.5, None, None, None,
                      None, ws)
    torch.cuda.synchronize()
    gv, ga = O.cfg_combine(vv, 5.0), O.cfg_combine(va, 5.0)
    exp_v = O.euler_update(xv[:nv], gv, 0.0, 0.25) if nv else xv
    exp_a = O.euler_update(xa[:na], ga, 0.0, 0.5) if na else xa
    np.testing.assert_allclose(Xv.cpu().numpy()[:max(nv, 1)], np.concatenate([exp_v, xv[nv:]])[:max(nv, 1)],
                               rtol=2e-6, atol=2e-6)
    np.testing.assert_allclose(Xa.cpu().numpy()[:max(na, 1)], np.concatenate([exp_a, xa[na:]])[:max(na, 1)],
                               rtol=2e-6, atol=2e-6)


def cache_host(dc, length):
    """Device cache -> the oracle's layout: per layer [br, length, H*d] keys and values (float32)."""
    k = dc.k[..., :length, :].float().cpu().numpy()    # [L, br, H, len, d]
    v = dc.v[..., :length].float().cpu().numpy()       # [L, br, H, d, len]
    L, br, H, n, d = k.shape
    return O.KVCache([k[l].transpose(0, 2, 1, 3).reshape(br, n, H * d) for l in range(L)],
                     [v[l].transpose(0, 3, 1, 2).reshape(br, n, H * d) for l in range(L)])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_evict_matches_oracle(gpu, tiny_oracle, dtype):
    """Window eviction on the GPU (one of three cached chunks dropped, positions moved back by one
    chunk of frames) against the oracle's eviction of the same cache contents, then a denoising
    step on the evicted cache against the oracle's step on its own evicted cache."""
    w, m, ckv = tiny_oracle
    Lq, Fc = w.chunk_tokens, w.frames_per_chunk
    print("kv-evict", dtype, flush=True)
    x1v, x1a, epv, epa = tiny_inputs(w)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache(4)
    for c in range(3):
        rig.append(dc, x1v[c], x1a[c], c * Fc)
    torch.cuda.synchronize()
    before = cache_host(dc, 3 * Lq)
    ref = O.KVCache([k.astype(np.float64) for k in before.k], [v.astype(np.float64) for v in before.v])
    O.kv_evict(w, ref, Lq, Fc)
    wam.wam_kv_evict(rig.m.cfg, dc.c, Lq, Fc)
    torch.cuda.synchronize()
    assert dc.length == 2 * Lq
    after = cache_host(dc, 2 * Lq)
    for l in range(w.layers):
        assert np.array_equal(after.v[l], ref.v[l])          # values only move
        scale = np.abs(before.k[l]).max()
        if dtype == "f32":
            assert np.abs(after.k[l] - ref.k[l]).max() <= 1e-6 * scale
        else:   # one rounding of the rotated key to bf16
            assert np.all(np.abs(after.k[l] - ref.k[l]) <= np.abs(ref.k[l]) * 2.0 ** -8 + 1e-6 * scale)
    # the next chunk, denoised at its position lowered by the shift
    xv = O.interpolate(x1v[2], epv[2], 0.4)
    xa = O.interpolate(x1a[2], epa[2], 0.4)
    gv, ga = rig.step(dc, 1, xv, xa, [0.4], [0.4], 2 * Fc)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    for c in range(3):
        O.kv_append(m, cache, ckv, x1v[c], x1a[c], c * Fc)
    O.kv_evict(w, cache, Lq, Fc)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, xv, xa, [0.4], [0.4], 1, 2 * Fc)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]


# Reuse decisions taken on real cosines of the tiny model (seeded inputs; the oracle's cosines of
# successive guided velocities lie in 0.994 .. 0.9988 on these grids). Each "decide" case's threshold
# sits where the oracle's run decides by the cosine (some later steps reuse, some do not), 1.5e-4 to
# 3e-4 from every cosine it compares. A decision is unique when both implementations' cosines lie on
# the same side of tau: the GPU first replays the oracle's mask and reports the cosines it compares
# along it; then, if every one is on the oracle's side, its own loop must take exactly the oracle's
# decisions. The cosines agree within 1e-4 in fp32; in bf16 the first-order bound is
# |d cos| <= (e_a + e_b) sin(theta) with e = 2e-2, the bf16 bar on the velocities.
_G8 = [k / 8 for k in range(9)]
_G6 = [0.0, 0.1, 0.25, 0.45, 0.7, 0.85, 1.0]
_REUSE_CASES = [("g8", _G8, 0.998012, -1, "decide"), ("g8", _G8, 0.997458, 1, "decide"),
                ("g6", _G6, 0.994261, 1, "decide"), ("g8", _G8, None, -1, "replay")]
_REUSE_REF = {}


def _oracle_reuse(tiny_oracle, name, grid, tau, max_reuse):
    w, m, ckv = tiny_oracle
    x1v, x1a, epv, epa = tiny_inputs(w)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)

    def dit(xv, xa, t):
        vb, ab = O.stack_forward(m, cache, ckv, xv, xa, [t], [t], 1, w.frames_per_chunk)
        return O.cfg_combine(vb, w.guidance), O.cfg_combine(ab, w.guidance)
    if tau is None:   # a threshold on top of an observed cosine: only the replay applies
        trace = []
        O.denoise_chunk(dit, epv[1], epa[1], grid, 1.5, trace=trace)
        tau = trace[0][1]
    trace = []
    xv, xa, calls, flags = O.denoise_chunk(dit, epv[1], epa[1], grid, tau, None if max_reuse < 0 else max_reuse,
                                           trace=trace)
    return tau, xv, xa, calls, flags, trace


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(_REUSE_CASES)))
def test_reuse_decisions_on_real_cosines(gpu, tiny_oracle, dtype, case):
    name, grid, tau0, max_reuse, path = _REUSE_CASES[case]
    if case not in _REUSE_REF:
        _REUSE_REF[case] = _oracle_reuse(tiny_oracle, name, grid, tau0, max_reuse)
    tau, ref_v, ref_a, n_ref, flags_ref, trace = _REUSE_REF[case]
    w = tiny_oracle[0]
    margin = min(abs(c - tau) for _, c in trace)
    sin_max = max(np.sqrt(max(0.0, 1.0 - c * c)) for _, c in trace)
    band = 1e-4 if dtype == "f32" else 2 * TOL["bf16"] * sin_max
    print("reuse", dtype, name, "tau %.6f" % tau, "max_reuse", max_reuse, "margin %.2e" % margin,
          "flags", "".join("R" if f else "." for f in flags_ref), flush=True)
    if path == "decide":   # the cosine really decides: some steps reuse and some do not after step 1
        assert margin > 1e-4 and any(flags_ref[2:]) and not all(flags_ref[2:])
    x1v, x1a, epv, epa = tiny_inputs(w)
    rig = Rig(w, dtype, gpu)
    dc = rig.cache()
    rig.append(dc, x1v[0], x1a[0], 0)
    br = rig.m.cfg.branches
    bufs = lambda: (torch.empty((br, w.video_tokens, w.patch_dim), device=gpu),  # noqa: E731
                    torch.empty((br, w.action_tokens, w.action_dim), device=gpu),
                    torch.empty(w.video_tokens * w.patch_dim, device=gpu),
                    torch.empty(w.action_tokens * w.action_dim, device=gpu), torch.empty(3, device=gpu))
    # the oracle's decisions replayed, with the cosines the GPU compares along them
    xv, xa = rig.f32(epv[1]), rig.f32(epa[1])
    calls, cos = wam.wam_denoise_chunk_replay(rig.m.cfg, rig.m.weights, dc.c, rig.ctx.c, xv, xa, grid, w.guidance,
                                              flags_ref, *bufs(), rig.ws, start_frame=w.frames_per_chunk)
    torch.cuda.synchronize()
    assert calls == n_ref
    ev, ea = rel_l2(xv.cpu().numpy(), ref_v), rel_l2(xa.cpu().numpy(), ref_a)
    dcos = max(abs(cos[k] - c) for k, c in trace)
    evaluated = dict(trace)
    assert all(np.isnan(cos[k]) for k in range(len(grid) - 1) if k not in evaluated)
    same_side = all((cos[k] > tau) == (c > tau) for k, c in trace)
    print("replayed: rel-L2 video %.2e action %.2e; max |cos_gpu - cos_oracle| %.2e (band %.1e); decisions %s"
          % (ev, ea, dcos, band, "unique" if same_side else "ambiguous"), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]
    assert dcos <= band
    if path == "decide" and dtype == "f32":
        assert same_side   # the margin exceeds the fp32 band
    if path == "decide" and same_side:   # the library's own decisions must be the oracle's
        xv2, xa2 = rig.f32(epv[1]), rig.f32(epa[1])
        calls2, flags = wam.wam_denoise_chunk(rig.m.cfg, rig.m.weights, dc.c, rig.ctx.c, xv2, xa2, grid, w.guidance,
                                              tau, *bufs(), rig.ws, start_frame=w.frames_per_chunk,
                                              max_consecutive_reuse=max_reuse)
        torch.cuda.synchronize()
        assert flags == list(flags_ref) and calls2 == n_ref
        # same decisions, same kernels in the same order: the same latents bit for bit
        assert np.array_equal(xv2.cpu().numpy(), xv.cpu().numpy())
        assert np.array_equal(xa2.cpu().numpy(), xa.cpu().numpy())
