"""Pins of the oracle's time modulation, output head, per-token timestep routing and video token
positions, each against values fixed outside the function under test:

* time MLP: a hand-built scalar case whose values are closed forms of the logistic function, so a
  dropped or misplaced SiLU changes them ("DreamZero (WAM) 模型架构" §2.3, input sequence: a
  sinusoidal time embedding feeds the modulation);
* the [6, D] modulation split, through the block: with a zero modulation projection the six slots
  are the bias's six consecutive D-blocks, and a block whose first (or second) norm scale is -1
  collapses to a closed form that names which slot is shift, scale and gate (same page, §2.3 single
  causal block: shift/scale modulation of each norm's output, gated residuals; a reading of the pages);
* output head: LN(h)(1 + scale_h) + shift_h with both shift and scale offset by e, pinned by row
  statistics (same page, §2.3 output split);
* per-token timesteps: video rows of chunk c take t_video[c], action rows t_action[c] (paper
  walk-through, DreamZero-Flash: decoupled video / action noise levels);
* video positions: raster order (frame, row, column) written out for grids with rows != columns,
  and the rotary bands each axis turns (a reading of the pages).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from synth.workloads import WORKLOADS


def _logistic(x):
    return 1.0 / (1.0 + math.exp(-x))


def test_time_mlp_silu_placement_scalar_case():
    # freq_dim 8, width 8. t = 1 gives s = 0 and the sinusoid [1, 1, 1, 1, 0, 0, 0, 0] exactly.
    # W1 = I, b1 = 0: SiLU(1) = logistic(1), SiLU(0) = 0. W2 = 2 I, b2 = 0.5: e = 2 SiLU(emb) + 0.5.
    # Wp = six stacked identities, bp = slot index / 10: e6[i] = SiLU(e) + i / 10.
    D = 8
    g = {"t_w1": np.eye(D), "t_b1": np.zeros(D), "t_w2": 2.0 * np.eye(D), "t_b2": np.full(D, 0.5),
         "t_wp": np.concatenate([np.eye(D)] * 6), "t_bp": np.repeat(np.arange(6) / 10.0, D)}
    e, e6 = O.time_modulation(1.0, g, 8, dt=np.float64)
    s1 = _logistic(1.0)                     # 0.7310585786300049
    e_hi, e_lo = 2.0 * s1 + 0.5, 0.5         # units 0..3 / 4..7
    np.testing.assert_allclose(e, [e_hi] * 4 + [e_lo] * 4, rtol=1e-15, atol=0)
    silu_hi, silu_lo = e_hi * _logistic(e_hi), e_lo * _logistic(e_lo)
    assert e6.shape == (6, D)
    for i in range(6):
        np.testing.assert_allclose(e6[i], np.array([silu_hi] * 4 + [silu_lo] * 4) + i / 10.0, rtol=1e-14, atol=0)
    # the values differ from every single-SiLU or no-SiLU placement
    assert abs(silu_hi - e_hi) > 0.1 and abs(e_hi - (2.0 + 0.5)) > 0.1


def _slot_setup(scale_slot, zero_gate_slot, seed):
    """Tiny one-layer model with a zero modulation projection: e6 = t_bp as six D-blocks, and every
    layer offset zero. Slot ``scale_slot`` is -1 (its norm's output is then exactly its shift), slot
    ``zero_gate_slot`` is 0; the others are random. Cross-attention output projection zeroed."""
    w = WORKLOADS[1].with_(layers=1)
    D = w.dim
    m = O.load_model(w, dt=np.float64)
    rng = np.random.default_rng(seed)
    slots = rng.standard_normal((6, D)) * 0.3
    slots[scale_slot] = -1.0
    slots[zero_gate_slot] = 0.0
    g = dict(m.g, t_wp=np.zeros_like(m.g["t_wp"]), t_bp=slots.reshape(-1).copy())
    lp = dict(m.layers[0], mod=np.zeros((6, D)), w_co=np.zeros((D, D)), b_co=np.zeros(D))
    T = w.chunk_tokens
    h = rng.standard_normal((w.branches, T, D))
    e6, _ = O.per_token_time(w, g, [0.3], [0.8], 1, np.float64)
    return w, g, lp, slots, h, e6


def test_modulation_slots_self_attention_closed_form():
    # scale1 = -1: the first norm's output is shift1 on every row, so q, k, v are the same on every
    # row and every value row (cached ones included) is v0 = shift1 Wv^T + bv. Attention then returns
    # v0 whatever the keys, and with gate2 = 0 and W_co = b_co = 0 the block is exactly
    # h + gate1 * (v0 Wo^T + bo). Swapping shift and scale, or any other slot order, breaks this.
    w, g, lp, slots, h, e6 = _slot_setup(scale_slot=1, zero_gate_slot=5, seed=3)
    D = w.dim
    Wv, bv = lp["w_qkv"][2 * D:], lp["b_qkv"][2 * D:]
    v0 = np.matmul(slots[0], Wv.T) + bv
    L0 = 2 * w.chunk_tokens
    rng = np.random.default_rng(5)
    ck = rng.standard_normal((w.branches, L0, D))                      # any keys
    cv = np.broadcast_to(v0, (w.branches, L0, D)).copy()
    ctx = rng.standard_normal((w.branches, w.ctx_len, D))
    pos = O.video_positions(w, 1, 4)
    out, _, vn = O.block_forward(w, lp, h, e6, ctx, ctx, ck, cv, 1, pos)
    np.testing.assert_allclose(vn, np.broadcast_to(v0, vn.shape), rtol=1e-12, atol=1e-12)
    expect = h + slots[2] * (np.matmul(v0, lp["w_o"].T) + lp["b_o"])
    np.testing.assert_allclose(out, expect, rtol=1e-11, atol=1e-11)
    # and the self-attention really contributes (gate1 is not zero)
    assert np.abs(out - h).max() > 1e-3


def test_modulation_slots_feed_forward_closed_form():
    # gate1 = 0 removes the self-attention, W_co = 0 the cross-attention; scale2 = -1 makes the second
    # norm's output shift2 on every row, so the block is h + gate2 * (GELU_tanh(shift2 W1^T + b1) W2^T + b2)
    # (GELU from torch).
    w, g, lp, slots, h, e6 = _slot_setup(scale_slot=4, zero_gate_slot=2, seed=4)
    rng = np.random.default_rng(6)
    D = w.dim
    ctx = rng.standard_normal((w.branches, w.ctx_len, D))
    z = np.zeros((w.branches, 0, D))
    out, _, _ = O.block_forward(w, lp, h, e6, ctx, ctx, z, z, 1, O.video_positions(w, 1, 0))
    u = torch.from_numpy(np.matmul(slots[3], lp["w_ff1"].T) + lp["b_ff1"])
    f = np.matmul(F.gelu(u, approximate="tanh").numpy(), lp["w_ff2"].T) + lp["b_ff2"]
    np.testing.assert_allclose(out, h + slots[5] * f, rtol=1e-11, atol=1e-11)
    assert np.abs(out - h).max() > 1e-3


def _head_model(head_mod, eps=1e-14):
    # width 64 with identity heads of 64 outputs (patch_dim 64, action_dim 64): the head returns
    # the modulated norm itself on every row.
    w = WORKLOADS[1].with_(dim=64, heads=1, head_dim=64, action_dim=64, eps=eps)
    g = {"head_mod": head_mod, "vo_w": np.eye(64), "vo_b": np.zeros(64), "ao_w": np.eye(64), "ao_b": np.zeros(64)}
    return w, g


def _rows(vv, va, w):
    """Per-branch [T, 64] rows of the head in token order (video rows, then action rows)."""
    return np.concatenate([vv, va], axis=1)


def test_head_modulation_takes_e_on_shift_and_scale():
    rng = np.random.default_rng(7)
    D = 64
    # head_mod = 0, e = a per-token constant c: each row has mean c (shift) and std 1 + c (scale)
    w, g = _head_model(np.zeros((2, D)))
    T = w.chunk_tokens
    c = np.linspace(-0.4, 1.7, T)
    e = np.repeat(c[:, None], D, axis=1)
    h = rng.standard_normal((2, T, D)) * 3 + 1
    vv, va = O.head_forward(w, g, h, e, 1)
    y = _rows(vv, va, w)
    np.testing.assert_allclose(y.mean(axis=-1), np.broadcast_to(c, (2, T)), atol=1e-12)
    np.testing.assert_allclose(y.std(axis=-1), np.broadcast_to(1 + c, (2, T)), rtol=1e-9)
    # e = 0, head_mod rows (s, k): row mean s, std 1 + k (row 0 shift, row 1 scale)
    w, g = _head_model(np.stack([np.full(D, 0.6), np.full(D, -0.3)]))
    vv, va = O.head_forward(w, g, h, np.zeros((T, D)), 1)
    y = _rows(vv, va, w)
    np.testing.assert_allclose(y.mean(axis=-1), 0.6, atol=1e-12)
    np.testing.assert_allclose(y.std(axis=-1), 0.7, rtol=1e-9)


def test_per_token_time_routes_video_and_action_rows():
    w = WORKLOADS[1].with_(layers=1)
    m = O.load_model(w, dt=np.float64)
    tv, ta = [0.2, 0.7], [0.9, 0.4]
    e6, e = O.per_token_time(w, m.g, tv, ta, 2, np.float64)
    Lv, Lq = w.video_tokens, w.chunk_tokens
    assert e6.shape == (2 * Lq, 6, w.dim) and e.shape == (2 * Lq, w.dim)
    tables = {}
    for c in range(2):
        for name, t, lo, hi in (("v", tv[c], c * Lq, c * Lq + Lv), ("a", ta[c], c * Lq + Lv, (c + 1) * Lq)):
            ref_e, ref_e6 = O.time_modulation(t, m.g, w.freq_dim, np.float64)
            assert np.array_equal(e6[lo:hi], np.broadcast_to(ref_e6, (hi - lo,) + ref_e6.shape))
            assert np.array_equal(e[lo:hi], np.broadcast_to(ref_e, (hi - lo,) + ref_e.shape))
            tables[(name, c)] = ref_e6
    keys = list(tables)
    for i in range(len(keys)):   # the four timesteps give four different tables
        for j in range(i + 1, len(keys)):
            assert np.abs(tables[keys[i]] - tables[keys[j]]).max() > 1e-6


def test_video_positions_raster_tables():
    w = WORKLOADS[1].with_(frames_per_chunk=1, grid_h=2, grid_w=3)
    expect = [(4, 0, 0), (4, 0, 1), (4, 0, 2), (4, 1, 0), (4, 1, 1), (4, 1, 2),
              (5, 0, 0), (5, 0, 1), (5, 0, 2), (5, 1, 0), (5, 1, 1), (5, 1, 2)]
    assert O.video_positions(w, 2, 4).tolist() == [list(p) for p in expect]
    w = WORKLOADS[1].with_(frames_per_chunk=2, grid_h=2, grid_w=1)
    assert O.video_positions(w, 1, 0).tolist() == [[0, 0, 0], [0, 1, 0], [1, 0, 0], [1, 1, 0]]


@pytest.mark.parametrize("token,band", [(3, 1), (1, 2), (6, 0)])
def test_video_positions_drive_their_rotary_bands(token, band):
    # 1 frame per chunk of 2 x 3 patches: token 3 is (frame s, row 1, col 0), token 1 (s, 0, 1) and
    # token 6 the first token of the next chunk (s + 1, 0, 0). With start frame s = 0, only the band of
    # the axis whose position is 1 turns: pairs 0..21 frame, 22..42 row, 43..63 column (d = 128).
    w = WORKLOADS[1].with_(frames_per_chunk=1, grid_h=2, grid_w=3)
    pos = O.video_positions(w, 2, 0)[token:token + 1]
    x = np.tile(np.array([1.0, 0.0]), 64)[None, None, :]
    y = O.apply_rope(x, pos, 128, 10000.0)[0, 0]
    bands = [(0, 22), (22, 43), (43, 64)]
    for b, (lo, hi) in enumerate(bands):
        moved = not np.array_equal(y[2 * lo:2 * hi], x[0, 0, 2 * lo:2 * hi])
        assert moved == (b == band)
    lo = bands[band][0]
    assert abs(y[2 * lo] - math.cos(1.0)) < 1e-15 and abs(y[2 * lo + 1] - math.sin(1.0)) < 1e-15
