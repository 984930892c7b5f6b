"""Model-level pins of the oracle on the tiny workload (width 256, 4 heads of 64, 2 frames of 8x8
patches + 24 action tokens, 32 text tokens), against invariants the pages fix:

* incremental chunk-by-chunk decoding with the KV cache equals one full-sequence pass under the
  chunk-causal mask (max abs diff <= 1e-5 in fp32) -- the noisy chunk sees clean earlier chunks
  and never future tokens (hyper.ai summary, 方法; paper walk-through, training objective);
* perturbing future-chunk tokens leaves earlier outputs bit-identical (same passages);
* shifting every frame position leaves the step unchanged (rotary positions are relative);
* zero gates remove the self-attention and FFN sub-layers exactly;
* CFG as a batch of 2 equals two single-branch passes;
* velocity reuse call counts at the threshold extremes (paper walk-through, DiT caching).
"""
import numpy as np
import pytest

import oracle as O
import synth
from synth.workloads import WORKLOADS, draw_named


@pytest.fixture(scope="module")
def tiny():
    w = WORKLOADS[1].with_(layers=2)
    m = O.load_model(w)
    txt = draw_named(w, -1, "txt")
    ctx = O.build_context(w, m.g, txt, None)
    ckv = [O.context_kv(w, lp, ctx) for lp in m.layers]
    x1v = [draw_named(w, -1, "x1_video_%d" % c) for c in range(3)]
    x1a = [draw_named(w, -1, "x1_action_%d" % c) for c in range(3)]
    epv = [draw_named(w, -1, "eps_video_%d" % c) for c in range(3)]
    epa = [draw_named(w, -1, "eps_action_%d" % c) for c in range(3)]
    return w, m, txt, ckv, x1v, x1a, epv, epa


def _full(w, m, ckv, xs_v, xs_a, tv, ta, start=0):
    e = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    return O.stack_forward(m, e, ckv, np.concatenate(xs_v), np.concatenate(xs_a), tv, ta, len(xs_v), start)


def test_incremental_equals_full_sequence(tiny):
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    Lv, La, Fc = w.video_tokens, w.action_tokens, w.frames_per_chunk
    xv2 = O.interpolate(x1v[2], epv[2], 0.5)
    xa2 = O.interpolate(x1a[2], epa[2], 0.3)
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    O.kv_append(m, cache, ckv, x1v[1], x1a[1], Fc)
    assert cache.length == 2 * (Lv + La)
    vv, va = O.stack_forward(m, cache, ckv, xv2, xa2, [0.5], [0.3], 1, 2 * Fc)
    fv, fa = _full(w, m, ckv, [x1v[0], x1v[1], xv2], [x1a[0], x1a[1], xa2], [1, 1, 0.5], [1, 1, 0.3])
    assert np.abs(fv[:, 2 * Lv:] - vv).max() <= 1e-5
    assert np.abs(fa[:, 2 * La:] - va).max() <= 1e-5
    # the cache matters: without it the chunk's velocity changes
    e = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    nv, _ = O.stack_forward(m, e, ckv, xv2, xa2, [0.5], [0.3], 1, 2 * Fc)
    assert np.abs(nv - vv).max() > 1e-3


def test_future_perturbation_bit_identical(tiny):
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    Lv, La = w.video_tokens, w.action_tokens
    a = _full(w, m, ckv, [x1v[0], epv[1]], [x1a[0], epa[1]], [1, 0.2], [1, 0.2])
    b = _full(w, m, ckv, [x1v[0], epv[1] * 7 + 3], [x1a[0], -epa[1]], [1, 0.9], [1, 0.6])
    assert np.array_equal(a[0][:, :Lv], b[0][:, :Lv])
    assert np.array_equal(a[1][:, :La], b[1][:, :La])
    assert not np.array_equal(a[0][:, Lv:], b[0][:, Lv:])


def test_frame_shift_invariance_without_action_tokens(tiny):
    # Rotary scores depend only on position differences, so with video tokens alone a common shift of
    # every frame index leaves the step unchanged up to rounding. Action tokens are not rotated, so a
    # video-action score depends on the absolute frame index and the invariance stops holding once
    # they are present (checked below as well).
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    w0 = w.with_(action_tokens=0)
    m0 = O.Model(w0, m.g, m.layers)
    Fc = w.frames_per_chunk
    outs = []
    for start in (0, 5):
        cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
        O.kv_append(m0, cache, ckv, x1v[0], x1a[0][:0], start)
        outs.append(O.stack_forward(m0, cache, ckv, epv[1], epa[1][:0], [0.3], [0.3], 1, start + Fc))
    np.testing.assert_allclose(outs[0][0], outs[1][0], atol=2e-5)
    outs = []
    for start in (0, 5):
        cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
        O.kv_append(m, cache, ckv, x1v[0], x1a[0], start)
        outs.append(O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.3], [0.3], 1, start + Fc))
    assert np.abs(outs[0][0] - outs[1][0]).max() > 1e-4


def test_frames_are_positions_not_order(tiny):
    # Placing the same chunk at a different frame offset relative to the cache changes the output
    # (the rotary positions are used at all), so the invariance above is not vacuous.
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    a = O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.0], [0.0], 1, 2)
    b = O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.0], [0.0], 1, 9)
    assert np.abs(a[0] - b[0]).max() > 1e-4


def test_zero_gates_remove_self_attention_and_ffn(tiny):
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    g = dict(m.g)
    g["t_wp"] = np.zeros_like(g["t_wp"])
    g["t_bp"] = np.zeros_like(g["t_bp"])
    layers = []
    for lp in m.layers:
        lp = dict(lp)
        mod = lp["mod"].copy()
        mod[2] = 0.0
        mod[5] = 0.0
        lp["mod"] = mod
        layers.append(lp)
    m0 = O.Model(w, g, layers)
    # with both gates zero the output cannot depend on the self-attention or FFN weights
    layers2 = []
    for lp in layers:
        lp = dict(lp)
        for k in ("w_qkv", "w_o", "w_ff1", "w_ff2", "b_o", "b_ff2"):
            lp[k] = lp[k] * 3.0 + 0.1
        layers2.append(lp)
    m1 = O.Model(w, g, layers2)
    e = O.KVCache.empty(len(layers), w.branches, w.dim)
    a = O.stack_forward(m0, e, ckv, epv[1], epa[1], [0.4], [0.4], 1, 0)
    b = O.stack_forward(m1, e, ckv, epv[1], epa[1], [0.4], [0.4], 1, 0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_cfg_batch_equals_single_branch_runs(tiny):
    w, m, txt, _, x1v, x1a, epv, epa = tiny
    full_ctx = O.build_context(w, m.g, txt, None)
    ckv2 = [O.context_kv(w, lp, full_ctx) for lp in m.layers]
    e = O.KVCache.empty(len(m.layers), 2, w.dim)
    both = O.stack_forward(m, e, ckv2, epv[0], epa[0], [0.3], [0.3], 1, 0)
    w1 = w.with_(branches=1)
    m1 = O.Model(w1, m.g, m.layers)
    for b in range(2):
        ctx_b = O.build_context(w1, m.g, txt[b:b + 1], None)
        ckv1 = [O.context_kv(w1, lp, ctx_b) for lp in m.layers]
        e1 = O.KVCache.empty(len(m.layers), 1, w.dim)
        one = O.stack_forward(m1, e1, ckv1, epv[0], epa[0], [0.3], [0.3], 1, 0)
        np.testing.assert_allclose(one[0][0], both[0][b], atol=1e-6)
        np.testing.assert_allclose(one[1][0], both[1][b], atol=1e-6)
    # the two branches do differ (different text features)
    assert np.abs(both[0][0] - both[0][1]).max() > 1e-4


def _dit_counter(w, m, ckv, cache, start):
    calls = []

    def dit(xv, xa, t):
        vb, ab = O.stack_forward(m, cache, ckv, xv, xa, [t], [t], 1, start)
        out = (O.cfg_combine(vb, w.guidance), O.cfg_combine(ab, w.guidance))
        calls.append((t, out))
        return out
    return dit, calls


def test_velocity_reuse_extremes(tiny):
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    grid = [k / 16 for k in range(17)]
    dit, calls = _dit_counter(w, m, ckv, cache, w.frames_per_chunk)
    _, _, n_a, flags_a = O.denoise_chunk(dit, epv[1], epa[1], grid, tau=1.5)
    assert n_a == 16 and len(calls) == 16 and not any(flags_a)
    dit, calls = _dit_counter(w, m, ckv, cache, w.frames_per_chunk)
    xv_b, xa_b, n_b, flags_b = O.denoise_chunk(dit, epv[1], epa[1], grid, tau=-1.5)
    assert n_b == 2 and len(calls) == 2 and flags_b == [False, False] + [True] * 14
    # after step 1 every update reuses v_1: x_16 = x_0 + v_0/16 + 15 v_1/16 for both modalities
    (_, (v0v, v0a)), (_, (v1v, v1a)) = calls
    np.testing.assert_allclose(xv_b, epv[1] + v0v / 16 + 15 * v1v / 16, atol=1e-5)
    np.testing.assert_allclose(xa_b, epa[1] + v0a / 16 + 15 * v1a / 16, atol=1e-5)
    # max_consecutive_reuse=1 alternates compute/reuse after step 1
    dit, calls = _dit_counter(w, m, ckv, cache, w.frames_per_chunk)
    _, _, n_c, flags_c = O.denoise_chunk(dit, epv[1], epa[1], grid, tau=-1.5, max_consecutive_reuse=1)
    assert flags_c == [False, False] + [True, False] * 7 and n_c == 9


def test_workload_shapes_match_pages():
    # Hyper-parameters printed on the pages (tests/golden/pages_hyperparams.txt, with citations).
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_hyperparams.txt")
    vals = {}
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split("=")
            vals[k.strip()] = int(v)
    w = WORKLOADS[3]
    assert w.layers == vals["layers"] and w.dim == vals["dim"] and w.heads == vals["heads"]
    assert w.head_dim == vals["head_dim"] and w.ffn_dim == vals["ffn_dim"]
    assert w.ctx_in_dim == vals["encoder_dim"] and w.action_tokens == vals["action_horizon"]
    assert w.ctx_text_len == vals["text_len"] and w.patch_dim == vals["latent_channels"] * 4
    assert w.action_dim == vals["droid_action_dim"]
    # 320x176 frames, 8x spatial VAE compression, 2x2 patches -> 20 x 11 patch grid
    assert (vals["frame_w"] // vals["vae_spatial"] // 2, vals["frame_h"] // vals["vae_spatial"] // 2) == (w.grid_w, w.grid_h)
    assert synth.BASE_SEED == vals["seed"]


def test_kv_evict_equals_appending_at_shifted_frames(tiny):
    # Layer-0 keys and values of a chunk depend on its own tokens and frame positions only (no
    # attention precedes them). So after evicting the first of three cached chunks and moving the
    # window back by one chunk of frames, the layer-0 rows of the two kept chunks must equal those
    # of the same chunks appended to an empty cache at frames lowered by that shift: keys up to the
    # rounding of one extra rotation, values exactly. Action rows are never rotated.
    w, m, _, ckv, x1v, x1a, _, _ = tiny
    Lq, Fc = w.chunk_tokens, w.frames_per_chunk
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    for c in range(3):
        O.kv_append(m, cache, ckv, x1v[c], x1a[c], c * Fc)
    ref = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    for c in (1, 2):
        O.kv_append(m, ref, ckv, x1v[c], x1a[c], (c - 1) * Fc)
    O.kv_evict(w, cache, Lq, Fc)
    assert cache.length == 2 * Lq
    assert np.array_equal(cache.v[0], ref.v[0])
    scale = np.abs(ref.k[0]).max()
    assert np.abs(cache.k[0] - ref.k[0]).max() <= 1e-5 * scale
    video = (np.arange(2 * Lq) % Lq) < w.video_tokens
    assert np.array_equal(cache.k[0][:, ~video], ref.k[0][:, ~video])


def test_kv_evict_without_shift_only_drops_rows(tiny):
    w, m, _, ckv, x1v, x1a, _, _ = tiny
    Lq, Fc = w.chunk_tokens, w.frames_per_chunk
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    for c in range(2):
        O.kv_append(m, cache, ckv, x1v[c], x1a[c], c * Fc)
    before = [k.copy() for k in cache.k], [v.copy() for v in cache.v]
    O.kv_evict(w, cache, Lq, 0)
    for l in range(len(m.layers)):
        assert np.array_equal(cache.k[l], before[0][l][:, Lq:])
        assert np.array_equal(cache.v[l], before[1][l][:, Lq:])


def test_rotary_composition_is_a_position_shift():
    # The eviction's extra rotation by (-s, 0, 0) equals rotating at the shifted position once.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 4, 64))
    pos = np.stack([rng.integers(0, 30, 40), rng.integers(0, 8, 40), rng.integers(0, 8, 40)], 1)
    twice = O.apply_rope(O.apply_rope(x, pos, 64, 1e4), np.tile([[-7, 0, 0]], (40, 1)), 64, 1e4)
    once = O.apply_rope(x, pos - np.array([7, 0, 0]), 64, 1e4)
    assert np.abs(twice - once).max() <= 1e-12


def _frame_causal(tiny):
    w, m = tiny[0], tiny[1]
    wf = w.with_(variant=synth.workloads.VARIANT_FRAME_CAUSAL)
    return wf, O.Model(wf, m.g, m.layers)


def test_frame_causal_mask_hides_later_frames_and_actions(tiny):
    # Frame-causal variant ([ARCH] §2.3 causal mask): inside a chunk, changing the second frame's
    # tokens cannot reach the first frame's outputs, and changing the action tokens cannot reach any
    # video output; both reach the action outputs. Under the adopted chunk-level mask they do reach.
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    wf, mf = _frame_causal(tiny)
    hw = w.grid_h * w.grid_w
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    O.kv_append(mf, cache, ckv, x1v[0], x1a[0], 0)
    base = O.stack_forward(mf, cache, ckv, epv[1], epa[1], [0.4], [0.4], 1, w.frames_per_chunk)
    xv2 = epv[1].copy()
    xv2[hw:] = xv2[hw:] * 3 - 1                       # second frame only
    f2 = O.stack_forward(mf, cache, ckv, xv2, epa[1], [0.4], [0.4], 1, w.frames_per_chunk)
    assert np.array_equal(base[0][:, :hw], f2[0][:, :hw])
    assert not np.array_equal(base[0][:, hw:], f2[0][:, hw:]) and not np.array_equal(base[1], f2[1])
    a2 = O.stack_forward(mf, cache, ckv, epv[1], -epa[1], [0.4], [0.4], 1, w.frames_per_chunk)
    assert np.array_equal(base[0], a2[0]) and not np.array_equal(base[1], a2[1])
    cache0 = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    O.kv_append(m, cache0, ckv, x1v[0], x1a[0], 0)
    c1 = O.stack_forward(m, cache0, ckv, epv[1], epa[1], [0.4], [0.4], 1, w.frames_per_chunk)
    c2 = O.stack_forward(m, cache0, ckv, xv2, epa[1], [0.4], [0.4], 1, w.frames_per_chunk)
    assert not np.array_equal(c1[0][:, :hw], c2[0][:, :hw])


def test_frame_causal_incremental_equals_full_sequence(tiny):
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    wf, mf = _frame_causal(tiny)
    Lv, La, Fc = w.video_tokens, w.action_tokens, w.frames_per_chunk
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    O.kv_append(mf, cache, ckv, x1v[0], x1a[0], 0)
    iv, ia = O.stack_forward(mf, cache, ckv, epv[1], epa[1], [0.3], [0.6], 1, Fc)
    fv, fa = _full(wf, mf, ckv, [x1v[0], epv[1]], [x1a[0], epa[1]], [1, 0.3], [1, 0.6])
    assert np.abs(fv[:, Lv:] - iv).max() <= 1e-5 and np.abs(fa[:, La:] - ia).max() <= 1e-5


def _embodiment_step(w, g, layers, ckv, x1v, x1a, epv, epa, e):
    me = O.Model(w, O.embodiment_params(g, e), layers)
    cache = O.KVCache.empty(len(layers), w.branches, w.dim)
    O.kv_append(me, cache, ckv, x1v[0], x1a[0], 0)
    return O.stack_forward(me, cache, ckv, epv[1], epa[1], [0.4], [0.4], 1, w.frames_per_chunk)


def test_embodiment_routing_encoder_and_decoder(tiny):
    """Architecture page §2.4: per-embodiment action encoder / decoder around a shared DiT. Embodiment
    0 is the default weights; a decoder-only difference leaves the video output bit-identical (the
    decoder runs after the DiT) and changes the action output; an encoder difference reaches the
    video rows through attention."""
    w, m, _, ckv, x1v, x1a, epv, epa = tiny
    assert O.embodiment_params(m.g, 0) is m.g
    rng = np.random.default_rng(11)
    g = dict(m.g)
    A, D = w.action_dim, w.dim
    # embodiment 1: own decoder, shared encoder; embodiment 2: own encoder, shared decoder
    g["ae_w_1"], g["ae_b_1"] = m.g["ae_w"], m.g["ae_b"]
    g["ao_w_1"] = (rng.standard_normal((A, D)) * 0.02).astype(np.float32)
    g["ao_b_1"] = (rng.standard_normal(A) * 0.02).astype(np.float32)
    g["ae_w_2"] = (rng.standard_normal((D, A)) * 0.02).astype(np.float32)
    g["ae_b_2"] = (rng.standard_normal(D) * 0.02).astype(np.float32)
    g["ao_w_2"], g["ao_b_2"] = m.g["ao_w"], m.g["ao_b"]
    v0, a0 = _embodiment_step(w, g, m.layers, ckv, x1v, x1a, epv, epa, 0)
    v1, a1 = _embodiment_step(w, g, m.layers, ckv, x1v, x1a, epv, epa, 1)
    v2, a2 = _embodiment_step(w, g, m.layers, ckv, x1v, x1a, epv, epa, 2)
    assert np.array_equal(v0, v1)
    assert not np.allclose(a0, a1)
    assert not np.array_equal(v0, v2) and not np.allclose(a0, a2)


def _img_setup(variant):
    w = WORKLOADS[1].with_(layers=2, ctx_img_len=16, variant=variant)
    m = O.load_model(w)
    txt = draw_named(w, -1, "txt")
    img = draw_named(w, -1, "img")
    return w, m, txt, img


def _step_with_ctx(w, m, ctx, x1v, x1a, epv, epa):
    ckv = [O.context_kv(w, lp, ctx) for lp in m.layers]
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    return O.stack_forward(m, cache, ckv, epv[1], epa[1], [0.4], [0.4], 1, w.frames_per_chunk)


def test_separate_image_attention_pins(tiny):
    """Image cross-attention variant (own image key / value projections, own softmax, outputs summed):
    with the image value projection zero the image branch adds exactly nothing, so the step equals the
    text-only model bit for bit; the image tokens form a set (permuting them changes nothing beyond
    rounding); and the variant differs from one softmax over the concatenated sequence."""
    _, _, _, _, x1v, x1a, epv, epa = tiny
    w, m, txt, img = _img_setup(8)
    layers0 = [dict(lp, w_cvi=np.zeros_like(lp["w_cvi"]), b_cvi=np.zeros_like(lp["b_cvi"])) for lp in m.layers]
    m0 = O.Model(w, m.g, layers0)
    v_zero, a_zero = _step_with_ctx(w, m0, O.build_context(w, m.g, txt, img), x1v, x1a, epv, epa)
    wt = w.with_(ctx_img_len=0, variant=0)
    mt = O.Model(wt, m.g, m.layers)
    v_txt, a_txt = _step_with_ctx(wt, mt, O.build_context(wt, m.g, txt, None), x1v, x1a, epv, epa)
    assert np.array_equal(v_zero, v_txt) and np.array_equal(a_zero, a_txt)
    v1, a1 = _step_with_ctx(w, m, O.build_context(w, m.g, txt, img), x1v, x1a, epv, epa)
    perm = np.random.default_rng(2).permutation(img.shape[0])
    v2, a2 = _step_with_ctx(w, m, O.build_context(w, m.g, txt, img[perm]), x1v, x1a, epv, epa)
    assert np.allclose(v1, v2, rtol=0, atol=1e-5 * np.abs(v1).max()) and np.allclose(a1, a2, rtol=0,
                                                                                    atol=1e-5 * np.abs(a1).max())
    wc = w.with_(variant=0)
    vc, ac = _step_with_ctx(wc, O.Model(wc, m.g, m.layers), O.build_context(wc, m.g, txt, img), x1v, x1a, epv, epa)
    assert not np.allclose(v1, vc, rtol=0, atol=1e-4 * np.abs(v1).max())


def test_state_rows_in_the_condition_sequence(tiny):
    """State rows (reading: one encoder Linear, rows appended to the condition sequence): cross
    attention treats the condition tokens as a set, so moving the state row to the front of the
    sequence changes nothing beyond rounding; a different observed state changes the step; a
    sequence whose last text row equals the state row's embedding (text made one row shorter) gives
    the same result as the state-row model."""
    _, _, _, _, x1v, x1a, epv, epa = tiny
    w = WORKLOADS[1].with_(layers=2, ctx_state_len=1)
    m = O.load_model(w)
    txt = draw_named(w, -1, "txt")
    st0, st1 = draw_named(w, -1, "state_0"), draw_named(w, -1, "state_1")

    def step(ctx, ww=w):
        ckv = [O.context_kv(ww, lp, ctx) for lp in m.layers]
        cache = O.KVCache.empty(ww.layers, ww.branches, ww.dim)
        O.kv_append(O.Model(ww, m.g, m.layers), cache, ckv, x1v[0], x1a[0], 0)
        return O.stack_forward(O.Model(ww, m.g, m.layers), cache, ckv, epv[1], epa[1], [0.4], [0.4], 1,
                               ww.frames_per_chunk)

    ctx = O.build_context(w, m.g, txt, None, st0)
    assert ctx.shape == (w.branches, w.ctx_len, w.dim)
    v0, a0 = step(ctx)
    front = np.concatenate([ctx[:, -1:], ctx[:, :-1]], axis=1)
    vf, af = step(front)
    assert np.allclose(v0, vf, rtol=0, atol=1e-5 * np.abs(v0).max()) and np.allclose(a0, af, rtol=0,
                                                                                    atol=1e-5 * np.abs(a0).max())
    v1, _ = step(O.build_context(w, m.g, txt, None, st1))
    assert not np.allclose(v0, v1, rtol=0, atol=1e-4 * np.abs(v0).max())
    # the state row is one more condition row: a text-only model with that row in place of its last
    # text row (text one shorter) is the same computation
    wt = w.with_(ctx_state_len=0, ctx_text_len=w.ctx_text_len + 1)
    ctx_t = np.concatenate([ctx[:, :-1], ctx[:, -1:]], axis=1)
    vt, at = step(ctx_t, wt)
    assert np.array_equal(v0, vt) and np.array_equal(a0, at)


def test_layer_major_passes_equal_sequential_calls(tiny):
    # stack_passes runs appends and steps together layer by layer (each layer's weights drawn once);
    # it must give exactly what kv_append / stack_forward give called one after another, and the lazily
    # drawn layers must be the eagerly drawn ones.
    w, m, txt, ckv, x1v, x1a, epv, epa = tiny
    Fc = w.frames_per_chunk
    cache = O.KVCache.empty(len(m.layers), w.branches, w.dim)
    O.kv_append(m, cache, ckv, x1v[0], x1a[0], 0)
    O.kv_append(m, cache, ckv, x1v[1], x1a[1], Fc)
    ref = O.stack_forward(m, cache, ckv, epv[2], epa[2], [0.35], [0.6], 1, 2 * Fc)
    ref2 = O.stack_forward(m, cache, ckv, np.concatenate([epv[0], epv[1]]), np.concatenate([epa[0], epa[1]]),
                           [0.2, 0.7], [0.4, 0.9], 2, 2 * Fc)
    lazy = O.load_model_lazy(w)
    for model in (m, lazy):
        ctx = O.build_context(w, model.g, txt, None)
        passes = [O.PassSpec(x1v[0], x1a[0], [1.0], [1.0], 1, 0, commit=True, heads=False),
                  O.PassSpec(x1v[1], x1a[1], [1.0], [1.0], 1, Fc, commit=True, heads=False),
                  O.PassSpec(epv[2], epa[2], [0.35], [0.6], 1, 2 * Fc),
                  O.PassSpec(np.concatenate([epv[0], epv[1]]), np.concatenate([epa[0], epa[1]]), [0.2, 0.7],
                             [0.4, 0.9], 2, 2 * Fc)]
        c2 = O.KVCache.empty(len(model.layers), w.branches, w.dim)
        seen = []
        outs = O.stack_passes(model, ctx, passes, cache=c2, progress=seen.append)
        assert seen == list(range(w.layers)) and outs[0] is None and outs[1] is None
        for got, want in ((outs[2], ref), (outs[3], ref2)):
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
        for l in range(w.layers):
            assert np.array_equal(c2.k[l], cache.k[l]) and np.array_equal(c2.v[l], cache.v[l])
