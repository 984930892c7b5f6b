"""Parity of the HIP path with the oracle at the benchmarked sizes, and of the single-block entry point.

* The 40-layer step at full width (5120, 40 heads of 128, FFN 13824), CFG batch 2, two committed
  clean chunks (928 cached tokens) and the timestep and noisy latents of bench.py's first step,
  against the oracle's own condition build, two appends and step (float32, layers drawn on demand);
  rel-L2 <= 2e-2 on video and action ("DreamZero (WAM) 模型架构" §5 hyper-parameter table, §2.3 the
  causal block stacked 40 times).
* The long-context geometry: three stitched views (11 x 60 patches, 1344 tokens per chunk), six
  committed chunks (8064 cached tokens), decoupled timesteps t_v = 1 - Beta(2, 1) and t_a ~ U(0, 1),
  full width with 2 layers.
* One full-width block through the stack call in bf16 (2e-2) and in the fp32 debug mode (1e-4).
* The step's kernels at full width (2 layers) twice on the same inputs: bit-identical outputs.
* wam_dit_block_fwd: incremental, two-chunk and committing chains at the tiny width (f32 and bf16),
  and at the full-width one-block shape with 2 branches and with 1 (the per-GPU share of a branch
  split), against oracle.block_forward on the same residual stream and modulation.

Long tests print progress lines past pytest's capture, so a minute of oracle work is never silent.
"""
import time

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


class Say:
    """Progress lines printed with pytest's capture suspended."""

    def __init__(self, capsys, name):
        self.capsys, self.name, self.t0 = capsys, name, time.time()

    def __call__(self, msg):
        with self.capsys.disabled():
            print("[%s %5.1fs] %s" % (self.name, time.time() - self.t0, msg), flush=True)


def f32dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def chunk_inputs(w, chunks):
    return ([draw_named(w, -1, "x1_video_%d" % c) for c in chunks], [draw_named(w, -1, "x1_action_%d" % c) for c in chunks],
            [draw_named(w, -1, "eps_video_%d" % c) for c in chunks], [draw_named(w, -1, "eps_action_%d" % c) for c in chunks])


class GpuRun:
    """Model, condition keys/values and KV cache of one workload on the GPU."""

    def __init__(self, w, dtype, dev, capacity_chunks, txt, img, packed=False):
        self.w, self.dtype, self.dev = w, dtype, dev
        self.m = DeviceModel(w, dtype, dev, packed=packed)
        self.ws = workspace(self.m.cfg, 2, dev)
        self.ctx = DeviceCtx(w, dtype, dev)
        wam.wam_ctx_build(self.m.cfg, self.m.weights, to_device(txt, dtype, dev),
                          to_device(img, dtype, dev) if img is not None else None, self.ctx.c, self.ws)
        self.cache = DeviceCache(w, capacity_chunks * w.chunk_tokens, dtype, dev)

    def append(self, xv, xa, start):
        wam.wam_kv_append(self.m.cfg, self.m.weights, self.cache.c, self.ctx.c, f32dev(xv, self.dev),
                          f32dev(xa, self.dev), start, self.ws)

    def step(self, xv, xa, tv, ta, start, n=1):
        w = self.w
        br = self.m.cfg.branches
        vv = torch.full((br, n * w.video_tokens, w.patch_dim), float("nan"), device=self.dev)
        va = torch.full((br, n * w.action_tokens, w.action_dim), float("nan"), device=self.dev)
        wam.wam_dit_stack_fwd(self.m.cfg, self.m.weights, self.cache.c, self.ctx.c, n, f32dev(xv, self.dev),
                              f32dev(xa, self.dev), tv, ta, start, vv, va, self.ws)
        torch.cuda.synchronize()
        return vv.cpu().numpy(), va.cpu().numpy()

    def e6(self, tv, ta):
        """Shared modulation [n][2][6][D] for chunk timesteps (video, action) from wam_time_embed."""
        t = [x for pair in zip(tv, ta) for x in pair]
        e = torch.empty((len(t), self.w.dim), device=self.dev)
        e6 = torch.empty((len(t), 6, self.w.dim), device=self.dev)
        wam.wam_time_embed(self.m.cfg, self.m.weights, t, e, e6, self.ws)
        return e6

    def rows(self, layer, r0, r1):
        """Keys / values of cache rows [r0, r1) of one layer in the oracle's layout [br, n, H*d]."""
        k = self.cache.k[layer, :, :, r0:r1, :].float().cpu().numpy()     # [br, H, n, d]
        v = self.cache.v[layer, :, :, :, r0:r1].float().cpu().numpy()     # [br, H, d, n]
        br, H, n, d = k.shape
        return k.transpose(0, 2, 1, 3).reshape(br, n, H * d), v.transpose(0, 3, 1, 2).reshape(br, n, H * d)


def _check_outputs(say, gv, ga, ref_v, ref_a, tol):
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    say("rel-L2 video %.3e action %.3e (bound %.0e)" % (ev, ea, tol))
    assert np.isfinite(gv).all() and np.isfinite(ga).all()
    assert ev <= tol and ea <= tol


@pytest.mark.timeout(1500)
def test_step_40_layers_cfg2_bf16_matches_oracle(gpu, capsys):
    """The benchmarked step: 40 layers, CFG batch 2, cache of 2 clean chunks (928 tokens), the noisy
    latents and timestep of bench.py's first step, with the fragment-packed projections bench.py uses
    (the unpacked copies deleted)."""
    w = WORKLOADS[3]
    say = Say(capsys, "40-layer step")
    Fc = w.frames_per_chunk
    t = float(synth.workloads.timesteps(w, 1)[0])
    x1v, x1a, _, _ = chunk_inputs(w, range(2))
    xv, xa = draw_named(w, -1, "eps_video_2"), draw_named(w, -1, "eps_action_2")
    txt, img = draw_named(w, -1, "txt"), draw_named(w, -1, "img")
    say("gpu: uploading %d layers, condition build, 2 appends, step at t = %.4f" % (w.layers, t))
    run = GpuRun(w, "bf16", gpu, 3, txt, img, packed=True)
    for c in range(2):
        run.append(x1v[c], x1a[c], c * Fc)
    assert run.cache.length == 2 * w.chunk_tokens
    gv, ga = run.step(xv, xa, [t], [t], 2 * Fc)
    del run
    torch.cuda.empty_cache()
    say("oracle: per layer its condition keys/values, 2 appends and the step")
    m = O.load_model_lazy(w)
    ctx = O.build_context(w, m.g, txt, img)
    passes = [O.PassSpec(x1v[0], x1a[0], [1.0], [1.0], 1, 0, commit=True, heads=False),
              O.PassSpec(x1v[1], x1a[1], [1.0], [1.0], 1, Fc, commit=True, heads=False),
              O.PassSpec(xv, xa, [t], [t], 1, 2 * Fc)]
    outs = O.stack_passes(m, ctx, passes, progress=lambda l: say("oracle layer %d/%d" % (l + 1, w.layers)))
    _check_outputs(say, gv, ga, outs[2][0], outs[2][1], TOL["bf16"])


@pytest.mark.timeout(600)
def test_full_width_step_run_to_run_bitwise(gpu, capsys):
    """The benchmarked step's kernels at full width (2 layers, CFG batch 2, 928 cached tokens, packed
    projections: the ten-wave attention, the split products and their finishes) give bit-identical
    outputs when the same step runs twice: every reduction has a fixed order."""
    w = WORKLOADS[3].with_(layers=2)
    say = Say(capsys, "full-width determinism")
    Fc = w.frames_per_chunk
    t = float(synth.workloads.timesteps(w, 1)[0])
    x1v, x1a, _, _ = chunk_inputs(w, range(2))
    xv, xa = draw_named(w, -1, "eps_video_2"), draw_named(w, -1, "eps_action_2")
    txt, img = draw_named(w, -1, "txt"), draw_named(w, -1, "img")
    say("gpu: 2 appends, the step twice at t = %.4f" % t)
    run = GpuRun(w, "bf16", gpu, 3, txt, img, packed=True)
    for c in range(2):
        run.append(x1v[c], x1a[c], c * Fc)
    gv1, ga1 = run.step(xv, xa, [t], [t], 2 * Fc)
    gv2, ga2 = run.step(xv, xa, [t], [t], 2 * Fc)
    del run
    torch.cuda.empty_cache()
    assert np.isfinite(gv1).all() and np.isfinite(ga1).all()
    assert np.array_equal(gv1, gv2) and np.array_equal(ga1, ga2)


@pytest.mark.timeout(1500)
def test_long_context_two_layers_decoupled_bf16_matches_oracle(gpu, capsys):
    """Three stitched views (1344 tokens per chunk), six committed chunks (8064 cached tokens), the
    decoupled timesteps of bench.py's first long-context step, full width, 2 layers, packed projections."""
    w = WORKLOADS[5].with_(layers=2)
    say = Say(capsys, "long context")
    Fc, C = w.frames_per_chunk, w.cache_chunks
    u = synth.uniform01(2, synth.tensor_key(w.id, -1, "timesteps"), stream=2)
    tv, ta = float(1.0 - np.sqrt(u[0])), float(u[1])   # sigma_v ~ Beta(2, 1) by the inverse CDF sqrt(u)
    x1v, x1a, _, _ = chunk_inputs(w, range(C))
    xv, xa = draw_named(w, -1, "eps_video_%d" % C), draw_named(w, -1, "eps_action_%d" % C)
    txt, img = draw_named(w, -1, "txt"), draw_named(w, -1, "img")
    say("gpu: %d appends of %d tokens, step at t_v = %.4f, t_a = %.4f" % (C, w.chunk_tokens, tv, ta))
    run = GpuRun(w, "bf16", gpu, C + 1, txt, img, packed=True)
    for c in range(C):
        run.append(x1v[c], x1a[c], c * Fc)
    assert run.cache.length == C * w.chunk_tokens == 8064
    gv, ga = run.step(xv, xa, [tv], [ta], C * Fc)
    del run
    torch.cuda.empty_cache()
    say("oracle")
    m = O.load_model_lazy(w)
    ctx = O.build_context(w, m.g, txt, img)
    passes = [O.PassSpec(x1v[c], x1a[c], [1.0], [1.0], 1, c * Fc, commit=True, heads=False) for c in range(C)]
    passes.append(O.PassSpec(xv, xa, [tv], [ta], 1, C * Fc))
    outs = O.stack_passes(m, ctx, passes, progress=lambda l: say("oracle layer %d/%d" % (l + 1, w.layers)))
    _check_outputs(say, gv, ga, outs[-1][0], outs[-1][1], TOL["bf16"])


@pytest.fixture(scope="module")
def block2():
    """Oracle side of the full-width one-block workload: one cached clean chunk, the current chunk at
    t ~ U(0, 1), its stack outputs, and block_forward on the embedded chunk."""
    w = WORKLOADS[2]
    Fc = w.frames_per_chunk
    m = O.load_model(w)
    txt, img = draw_named(w, -1, "txt"), draw_named(w, -1, "img")
    ctx = O.build_context(w, m.g, txt, img)
    ckv = [O.context_kv(w, lp, ctx) for lp in m.layers]
    x1v, x1a, epv, epa = chunk_inputs(w, range(2))
    t = float(synth.workloads.timesteps(w, 1)[0])
    xv1, xa1 = O.interpolate(x1v[1], epv[1], t), O.interpolate(x1a[1], epa[1], t)
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    ref = O.stack_forward(m, cache, ckv, xv1, xa1, [t], [t], 1, Fc)
    e6, _ = O.per_token_time(w, m.g, [t], [t], 1, np.float32)
    h0 = O.embed_tokens(m.g, xv1, xa1, w, 1)
    h = np.ascontiguousarray(np.broadcast_to(h0[None], (w.branches,) + h0.shape), dtype=np.float32)
    hb, kb, vb = O.block_forward(w, m.layers[0], h, e6, ckv[0][0], ckv[0][1], cache.k[0], cache.v[0], 1,
                                 O.video_positions(w, 1, Fc))
    return dict(w=w, t=t, txt=txt, img=img, x1v=x1v, x1a=x1a, xv1=xv1, xa1=xa1, ref=ref, h=h, hb=hb, kb=kb, vb=vb)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype,packed", [("bf16", False), ("f32", False), ("bf16", True)])
def test_full_width_block(gpu, capsys, block2, dtype, packed):
    """One Wan-14B-sized block through the stack call (769 condition tokens, one cached chunk of 464
    tokens, CFG batch 2) against the float32 oracle: 2e-2 in bf16 (unpacked or packed projections),
    1e-4 in the fp32 debug mode."""
    b = block2
    w, Fc = b["w"], b["w"].frames_per_chunk
    say = Say(capsys, "full-width block %s%s" % (dtype, " packed" if packed else ""))
    run = GpuRun(w, dtype, gpu, 2, b["txt"], b["img"], packed=packed)
    run.append(b["x1v"][0], b["x1a"][0], 0)
    gv, ga = run.step(b["xv1"], b["xa1"], [b["t"]], [b["t"]], Fc)
    _check_outputs(say, gv, ga, b["ref"][0], b["ref"][1], TOL[dtype])


# Full-width low-precision bound. At this width the MXFP8 block is ill-conditioned against changes
# of its projection inputs at bf16's precision: one such change flips about 1.5% of the fp8 codes by
# one step, and on the oracle alone rounding the six projection inputs to bf16 (at most 2^-9 relative)
# moves this block's MXFP8 output by 4.7e-2 (video) / 5.8e-2 (action), against 6.4e-2 / 7.4e-2 for
# the whole quantisation. The library's bf16 path perturbs every stored activation by as much, so the
# bound is twice that sensitivity; and the output must lie closer to the quantised oracle than the
# quantisation moves it (at most 0.85 of that distance), which a path that skipped or misplaced the
# quantisation (ratio about 1 or more) fails.
MX_FULL_TOL = 1e-1
MX_FULL_RATIO = 0.85


@pytest.mark.timeout(900)
@pytest.mark.parametrize("precision", [synth.workloads.PRECISION_MXFP8, synth.workloads.PRECISION_MXFP4W])
def test_full_width_block_low_precision(gpu, capsys, block2, precision):
    """The one-block full-width workload with the six projections in MXFP8 (or MXFP4 weights): at
    this width the K = 5120 / 13824 products split over K and their partials take the fused finish
    (which also writes the quantised copy of the next projection's input), a path only full-width
    shapes reach. Against the oracle with the same quantised projections."""
    b = block2
    w = b["w"].with_(precision=precision)
    Fc = w.frames_per_chunk
    say = Say(capsys, "full-width block precision %d" % precision)
    run = GpuRun(w, "bf16", gpu, 2, b["txt"], b["img"])
    run.append(b["x1v"][0], b["x1a"][0], 0)
    gv, ga = run.step(b["xv1"], b["xa1"], [b["t"]], [b["t"]], Fc)
    del run
    torch.cuda.empty_cache()
    m = O.load_model(w)
    ctx = O.build_context(w, m.g, b["txt"], b["img"])
    ckv = [O.context_kv(w, lp, ctx) for lp in m.layers]
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, b["x1v"][0], b["x1a"][0], 0)
    ref_v, ref_a = O.stack_forward(m, cache, ckv, b["xv1"], b["xa1"], [b["t"]], [b["t"]], 1, Fc)
    nat_v, nat_a = b["ref"]
    qv, qa = rel_l2(ref_v, nat_v), rel_l2(ref_a, nat_a)
    say("to the unquantised oracle: video %.3e action %.3e; oracle quantised to unquantised: video %.3e "
        "action %.3e" % (rel_l2(gv, nat_v), rel_l2(ga, nat_a), qv, qa))
    _check_outputs(say, gv, ga, ref_v, ref_a, MX_FULL_TOL)
    assert rel_l2(gv, ref_v) <= MX_FULL_RATIO * qv and rel_l2(ga, ref_a) <= MX_FULL_RATIO * qa


@pytest.mark.timeout(900)
@pytest.mark.parametrize("branches,packed", [(2, False), (1, False), (2, True)])
def test_block_fwd_full_width_bf16(gpu, capsys, block2, branches, packed):
    """wam_dit_block_fwd at the full-width one-block shape (the entry point behind the one-block timing),
    with the embedded current chunk as residual stream and the modulation from wam_time_embed,
    committing its keys/values. One branch is the conditional branch of the CFG pair (the branches
    never mix: the oracle's batch of 2 equals two single-branch runs)."""
    b = block2
    w = b["w"].with_(branches=branches)
    Fc, Lq, D = w.frames_per_chunk, w.chunk_tokens, w.dim
    say = Say(capsys, "block_fwd full width br=%d%s" % (branches, " packed" if packed else ""))
    run = GpuRun(w, "bf16", gpu, 2, b["txt"][:branches], b["img"], packed=packed)
    run.append(b["x1v"][0], b["x1a"][0], 0)
    e6 = run.e6([b["t"]], [b["t"]])
    h = b["h"][:branches]
    hd = f32dev(h, gpu)
    wam.wam_dit_block_fwd(run.m.cfg, run.m.blocks[0], 0, run.cache.c, run.ctx.c, hd, e6, 1, Fc, run.ws, commit=True)
    torch.cuda.synchronize()
    assert run.cache.length == 2 * Lq
    out = hd.cpu().numpy()
    k, v = run.rows(0, Lq, 2 * Lq)
    eh = rel_l2(out - h, b["hb"][:branches] - h)
    ek, evv = rel_l2(k, b["kb"][:branches]), rel_l2(v, b["vb"][:branches])
    say("rel-L2 block update %.3e, keys %.3e, values %.3e" % (eh, ek, evv))
    assert np.isfinite(out).all()
    assert eh <= TOL["bf16"] and ek <= TOL["bf16"] and evv <= TOL["bf16"]


@pytest.fixture(scope="module")
def tiny2():
    w = WORKLOADS[1].with_(layers=2)
    m = O.load_model(w)
    txt = draw_named(w, -1, "txt")
    ckv = [O.context_kv(w, lp, O.build_context(w, m.g, txt, None)) for lp in m.layers]
    x1v, x1a, epv, epa = chunk_inputs(w, range(3))
    cache = O.KVCache.empty(w.layers, w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    return w, m, txt, ckv, cache, x1v, x1a, epv, epa


def _residual(w, n, seed):
    return synth.fill((w.branches, n * w.chunk_tokens, w.dim), synth.tensor_key(w.id, -1, "block-h-%d" % seed),
                      "normal", 1.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layer,n,tv,ta", [(1, 1, [0.45], [0.45]), (0, 2, [0.3, 0.6], [0.5, 0.8])])
def test_block_fwd_tiny_matches_oracle(gpu, tiny2, dtype, layer, n, tv, ta):
    """One block over the committed chunk and n current chunks (n = 2: the chunk-causal full-sequence
    mode), decoupled timesteps, without commit: h, this call's key / value rows, the length."""
    w, m, txt, ckv, cache, x1v, x1a, epv, epa = tiny2
    Fc, Lq = w.frames_per_chunk, w.chunk_tokens
    print("block_fwd tiny", dtype, layer, n, flush=True)
    h = _residual(w, n, layer)
    e6, _ = O.per_token_time(w, m.g, tv, ta, n, np.float32)
    hb, kb, vb = O.block_forward(w, m.layers[layer], h, e6, ckv[layer][0], ckv[layer][1], cache.k[layer],
                                 cache.v[layer], n, O.video_positions(w, n, Fc))
    run = GpuRun(w, dtype, gpu, 3, txt, None)
    run.append(x1v[0], x1a[0], 0)
    hd = f32dev(h, gpu)
    wam.wam_dit_block_fwd(run.m.cfg, run.m.blocks[layer], layer, run.cache.c, run.ctx.c, hd, run.e6(tv, ta), n, Fc,
                          run.ws)
    torch.cuda.synchronize()
    assert run.cache.length == Lq
    out = hd.cpu().numpy()
    k, v = run.rows(layer, Lq, (n + 1) * Lq)
    errs = rel_l2(out - h, hb - h), rel_l2(k, kb), rel_l2(v, vb)
    print("rel-L2 block update %.3e keys %.3e values %.3e" % errs, flush=True)
    assert max(errs) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_fwd_commit_chain_then_step(gpu, tiny2, dtype):
    """Blocks run one by one with commit on the last: the length advances once, every layer's rows
    hold that chain's keys / values, and a following step uses them as cached context."""
    w, m, txt, ckv, cache, x1v, x1a, epv, epa = tiny2
    Fc, Lq = w.frames_per_chunk, w.chunk_tokens
    print("block_fwd commit chain", dtype, flush=True)
    h = _residual(w, 1, 7)
    e6, _ = O.per_token_time(w, m.g, [1.0], [1.0], 1, np.float32)
    pos = O.video_positions(w, 1, Fc)
    ref_cache = O.KVCache([k.copy() for k in cache.k], [v.copy() for v in cache.v])
    hr = h
    for l in range(w.layers):
        hr, kn, vn = O.block_forward(w, m.layers[l], hr, e6, ckv[l][0], ckv[l][1], cache.k[l], cache.v[l], 1, pos)
        ref_cache.k[l] = np.concatenate([ref_cache.k[l], kn], axis=1)
        ref_cache.v[l] = np.concatenate([ref_cache.v[l], vn], axis=1)
    ref_v, ref_a = O.stack_forward(m, ref_cache, ckv, epv[2], epa[2], [0.4], [0.4], 1, 2 * Fc)

    run = GpuRun(w, dtype, gpu, 3, txt, None)
    run.append(x1v[0], x1a[0], 0)
    hd = f32dev(h, gpu)
    e6d = run.e6([1.0], [1.0])
    for l in range(w.layers):
        wam.wam_dit_block_fwd(run.m.cfg, run.m.blocks[l], l, run.cache.c, run.ctx.c, hd, e6d, 1, Fc, run.ws,
                              commit=(l == w.layers - 1))
        assert run.cache.length == (2 if l == w.layers - 1 else 1) * Lq
    torch.cuda.synchronize()
    assert rel_l2(hd.cpu().numpy() - h, hr - h) <= TOL[dtype]
    for l in range(w.layers):
        k, v = run.rows(l, Lq, 2 * Lq)
        assert rel_l2(k, ref_cache.k[l][:, Lq:]) <= TOL[dtype] and rel_l2(v, ref_cache.v[l][:, Lq:]) <= TOL[dtype]
    gv, ga = run.step(epv[2], epa[2], [0.4], [0.4], 2 * Fc)
    ev, ea = rel_l2(gv, ref_v), rel_l2(ga, ref_a)
    print("step after the chain: rel-L2 video %.3e action %.3e" % (ev, ea), flush=True)
    assert ev <= TOL[dtype] and ea <= TOL[dtype]
