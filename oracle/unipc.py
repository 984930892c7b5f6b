"""UniPC multistep solver for the flow-matching denoising loop (oracle).

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may import it.

[WS1] ("DreamZero 单卡推理", architecture table and compile notes) names UniPC as the
scheduler's solver but prints no formula. The steps below restate the published method
(Zhao et al. 2023, "UniPC: a unified predictor-corrector framework for fast sampling of
diffusion models": the predictor UniP-p and corrector UniC-p in data-prediction form, with
B(h) = e^h - 1) for this repository's time convention, in the paper's notation:

* x_t = alpha_t x1 + sigma_t eps with alpha_t = t, sigma_t = 1 - t; half log-SNR
  lambda_t = log(alpha_t / sigma_t); the model's data prediction is m = x + sigma_t v
  (v the guided velocity, so that x1 - eps = v);
* one step from s to t: h = lambda_t - lambda_s, earlier outputs at s_j with
  r_j = (lambda_{s_j} - lambda_s) / h and D_j = (m_{s_j} - m_s) / r_j;
* h_phi_1 = e^{-h} - 1 and h_phi_{k+1} = h_phi_k / (-h) - 1/k!  (so h_phi_k = (-h) phi_k(-h));
* the coefficients rho solve sum_j rho_j r_j^(k-1) = h_phi_{k+1} k! / B_h, k = 1 .. (number of D);
* x_t = (sigma_t / sigma_s) x_s - alpha_t h_phi_1 m_s - alpha_t B_h sum_j rho_j D_j.

The predictor of order p uses m_s and p - 1 earlier outputs; the corrector of the same order adds
the output at the new point (r = 1, D = m_t - m_s), is applied once that output exists, and
replaces the predicted state while the output itself (taken at the predicted state) is kept.

Readings (no formula on the pages): order 2 by default; a step from t = 0 or to t = 1 (where
lambda is infinite) and the first step after one from t = 0 are taken at order 1 (the limits
e^{-h} -> 0 are exact there, and the order-1 predictor equals the Euler step); with velocity
reuse, a step whose velocity is reused forms its data prediction from the reused velocity and
skips the corrector (no fresh model output at that point).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .dit import cosine_fp64

Array = np.ndarray


def exp_neg_h(t_s: float, t_t: float) -> float:
    """e^{-h} for a step from s to t: (alpha_s sigma_t) / (sigma_s alpha_t); 0 when s = 0 or t = 1."""
    return (t_s * (1.0 - t_t)) / ((1.0 - t_s) * t_t)


def half_log_snr(t: float) -> float:
    return math.log(t / (1.0 - t))


def update_weights(t_t: float, t_hist: Sequence[float], corrector: bool) -> Tuple[float, List[float]]:
    """Weights of one UniPC update: x_new = a x_s + sum_i w_i m_i.

    ``t_hist`` = times of the outputs used, newest first (t_s, t_{s_1}, ...); the order is
    len(t_hist). With ``corrector`` the output at t_t is used too and its weight comes last.
    """
    t_s = t_hist[0]
    sig_s, sig_t, al_t = 1.0 - t_s, 1.0 - t_t, t_t
    e = exp_neg_h(t_s, t_t)
    hh = math.log(e) if e > 0.0 else -math.inf            # -h
    h_phi = [e - 1.0]                                        # h_phi_1
    for k in range(1, len(t_hist) + 1):
        h_phi.append(h_phi[-1] / hh - 1.0 / math.factorial(k))
    b_h = e - 1.0                                            # B(h) = e^h - 1 (data prediction: e^{-h} - 1)
    # r of the earlier outputs, then r = 1 for the corrector's new point
    rs = []
    if len(t_hist) > 1:
        h = -hh
        lam_s = half_log_snr(t_s)
        rs = [(half_log_snr(tj) - lam_s) / h for tj in t_hist[1:]]
    if corrector:
        rs.append(1.0)
    a = sig_t / sig_s
    w = [-al_t * h_phi[0]] + [0.0] * len(rs)
    if rs:
        n = len(rs)
        R = np.array([[r ** k for r in rs] for k in range(n)], dtype=np.float64)
        rhs = np.array([h_phi[k + 1] * math.factorial(k + 1) / b_h for k in range(n)], dtype=np.float64)
        rho = np.linalg.solve(R, rhs)
        for j, (r, p) in enumerate(zip(rs, rho)):
            c = -al_t * b_h * p / r                          # weight of the output behind D_j
            w[j + 1] += c
            w[0] -= c                                        # D_j subtracts m_s
    return a, w


def step_order(grid: Sequence[float], k: int, order: int) -> int:
    """Order of the predictor of step k (grid[k] -> grid[k+1]), readings above."""
    if grid[k] <= 0.0 or grid[k + 1] >= 1.0:
        return 1
    usable = 1
    while usable < order and k - usable >= 0 and grid[k - usable] > 0.0:
        usable += 1
    return usable


def denoise_chunk_unipc(dit, x_video: Array, x_action: Array, grid: Sequence[float], tau: float,
                        max_consecutive_reuse: Optional[int] = None, order: int = 2, corrector: bool = True):
    """UniPC loop with CFG-guided velocities and velocity reuse ([WS1] dynamic16; [N569] DiT caching).

    dit(x_video, x_action, t) -> guided (v_video, v_action). The reuse rule is the Euler loop's
    (a reading of the pages). Without ``corrector`` only the predictor runs (order 1 is then the Euler loop).
    Returns (x_video, x_action, number of DiT calls, per-step reuse flags).
    """
    assert all(b > a for a, b in zip(grid[:-1], grid[1:])) and grid[0] >= 0.0 and grid[-1] <= 1.0
    nv = x_video.size
    x = np.concatenate([x_video.ravel(), x_action.ravel()])
    dt = x.dtype
    ms: List[Array] = []          # data predictions, newest last
    x_prev: Optional[Array] = None
    prev_order = 0
    computed: List[Tuple[Array, Array]] = []
    calls, consecutive, flags = 0, 0, []
    for k in range(len(grid) - 1):
        t = grid[k]
        reuse = False
        if k >= 2 and len(computed) >= 2:
            c = cosine_fp64(computed[-1][0], computed[-2][0])
            if c > tau and (max_consecutive_reuse is None or consecutive < max_consecutive_reuse):
                reuse = True
        if reuse:
            vv, va = computed[-1]
            consecutive += 1
        else:
            vv, va = dit(x[:nv].reshape(x_video.shape), x[nv:].reshape(x_action.shape), t)
            computed.append((vv, va))
            calls += 1
            consecutive = 0
        flags.append(reuse)
        v = np.concatenate([vv.ravel(), va.ravel()]).astype(dt)
        m = x + dt.type(1.0 - t) * v
        if corrector and k >= 1 and not reuse:
            # corrector of step k-1 with the fresh output at t_k, same order as its predictor
            hist = [grid[k - 1 - j] for j in range(prev_order)]
            a, w = update_weights(t, hist, corrector=True)
            xs = dt.type(a) * x_prev
            for j in range(prev_order):
                xs = xs + dt.type(w[j]) * ms[-1 - j]
            x = xs + dt.type(w[-1]) * m
        ms.append(m)
        p = step_order(grid, k, order)
        a, w = update_weights(grid[k + 1], [grid[k - j] for j in range(p)], corrector=False)
        x_prev = x
        xn = dt.type(a) * x
        for j in range(p):
            xn = xn + dt.type(w[j]) * ms[-1 - j]
        x = xn
        prev_order = p
    return x[:nv].reshape(x_video.shape), x[nv:].reshape(x_action.shape), calls, flags
