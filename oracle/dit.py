"""Plain NumPy oracle of the chunk-causal joint video+action DiT denoise step.

TEST INFRASTRUCTURE ONLY: see ``oracle/__init__.py`` for who may import it.

Sources (titles of the pages; sections named, never quoted):
  [ARCH]  "DreamZero (WAM) 模型架构" (vla-model-architecture.pages.dev): §2.1
          encoders, §2.3 Causal WAN DiT (input sequence construction, single
          causal DiT block, output split, causal mask), §2.4 multi-embodiment
          action linears, §3 training pipeline (flow-matching interpolation),
          §4 inference pipeline (encode once, iterative denoise loop).
  [WS1]   "DreamZero 单卡推理" (PhyAI ws1 docs): architecture table (DiT runner
          keeps the attention KV; scheduler owns reference KV, CFG branches, DiT
          calls and the update), request format (negative prompt for CFG,
          512 text tokens), continuous requests (frame position, KV reset),
          Fixed4 vs dynamic16 (DiT re-run only when the prediction changes).
  [HYPER] hyper.ai summary of arXiv 2602.15922, "方法": chunked autoregressive
          generation, mask letting the noisy chunk see clean earlier chunks and
          never future tokens, KV-cache replacement by real observations,
          DreamZero-Flash decoupled schedules.
  [N569]  paper walk-through "World Action Models are Zero-shot Policies"
          (ai.n569.com): training objective (shared timestep, teacher forcing,
          joint velocity), inference (KV cache + observation feedback),
          real-time optimisations (CFG in parallel, DiT caching by cosine
          similarity of successive velocities, DreamZero-Flash Beta schedule).

Readings where the pages are silent, ambiguous or garbled are stated at the
function that takes them.

Conventions: time t in [0, 1], t = 0 pure noise, t = 1 clean;
x_t = t*x1 + (1-t)*eps; velocity target x1 - eps; Euler x += (t_next - t)*v.
Linear weights are [out, in] (y = x W^T + b). All arithmetic runs in ``dt``
(float32 by default, float64 on request); softmax is exp(S - rowmax)/sum.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

Array = np.ndarray


# ----------------------------------------------------------------------------------------------
# Elementary operations. Each is the textbook definition written out.
# ----------------------------------------------------------------------------------------------

def silu(x: Array) -> Array:
    """SiLU(x) = x * sigmoid(x) ([ARCH] §2.3: time embedding MLP; Wan-style, a reading of the pages)."""
    return x / (x.dtype.type(1) + np.exp(-x))


def gelu_tanh(x: Array) -> Array:
    """GELU with the tanh approximation: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    one = x.dtype.type(1)
    c = x.dtype.type(math.sqrt(2.0 / math.pi))
    return x.dtype.type(0.5) * x * (one + np.tanh(c * (x + x.dtype.type(0.044715) * x * x * x)))


def layer_norm(x: Array, eps: float, weight: Optional[Array] = None, bias: Optional[Array] = None) -> Array:
    """LayerNorm over the last axis, biased variance: (x - mean) / sqrt(var + eps) [* w + b].

    Reading: the block norms are LayerNorm (the running implementation's kernel policy on
    [WS1] names LayerNorm), not the RMSNorm drawn on [ARCH] §2.3.
    """
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    y = xc / np.sqrt(var + x.dtype.type(eps))
    if weight is not None:
        y = y * weight
    if bias is not None:
        y = y + bias
    return y


def rms_norm(x: Array, eps: float, gain: Optional[Array] = None) -> Array:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) [* g]."""
    ms = (x * x).mean(axis=-1, keepdims=True)
    y = x / np.sqrt(ms + x.dtype.type(eps))
    if gain is not None:
        y = y * gain
    return y


def linear(x: Array, w: Array, b: Optional[Array] = None) -> Array:
    """y = x W^T + b with W stored [out, in]."""
    y = x @ w.T
    if b is not None:
        y = y + b
    return y


def project(w, x: Array, W: Array, b: Optional[Array] = None) -> Array:
    """A block projection y = x W^T + b. With MXFP8 precision (1; the low-precision projections of
    [N569] real-time optimisations; formats and block rule in ``oracle.mx``) the rows of x and of W
    are first quantised along the input features and the product is taken of the quantised values,
    exactly (then cast back to the dtype of x); precision 2 quantises W to MXFP4 instead.
    Reading: the low-precision projections belong to the bf16 data type, whose activations are stored
    as bf16 rows; the rows the quantiser reads are those bf16 values, so x is rounded to bf16 first."""
    prec = getattr(w, "precision", 0)
    if prec not in (1, 2):
        return linear(x, W, b)
    from .mx import mx_linear, mx_quantize, round_bf16
    w_fmt = "e2m1" if prec == 2 else "e4m3"   # precision 2: MXFP4 weights, MXFP8 activations
    lead = x.shape[:-1]
    xc, xs = mx_quantize(round_bf16(x.reshape(-1, x.shape[-1])).astype(np.float64))
    wc, ws = mx_quantize(W.astype(np.float64), fmt=w_fmt)
    y = mx_linear(xc, xs, wc, ws, None if b is None else b.astype(np.float64), w_fmt=w_fmt)
    return y.reshape(lead + (W.shape[0],)).astype(x.dtype)


def modulated_norm(x: Array, shift: Array, scale: Array, eps: float, rms: bool = False) -> Array:
    """adaLN: LN(x) (1 + scale) + shift ([ARCH] §2.3 single block: the normed input is modulated
    by shift and scale from the time embedding; reading: scale enters as 1 + scale). With
    ``rms`` (the RMSNorm variant drawn on [ARCH] §2.3) the normalisation is RMSNorm."""
    n = rms_norm(x, eps) if rms else layer_norm(x, eps)
    return n * (x.dtype.type(1) + scale) + shift


def uses_rms(w) -> bool:
    """The RMSNorm variant: every block norm and the head norm normalise by the RMS (no mean)."""
    return bool(getattr(w, "variant", 0) & 2)


def softmax_rows(s: Array) -> Array:
    """exp(s - rowmax) / rowsum over the last axis. Entries equal to -inf get exactly 0."""
    m = s.max(axis=-1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=-1, keepdims=True)


def attention(q: Array, k: Array, v: Array, visible: Optional[Array] = None) -> Array:
    """Scaled dot-product attention per head.

    q [H, Lq, d], k [H, Lk, d], v [H, Lk, d]; ``visible`` [Lq, Lk] bool or None.
    S = q k^T / sqrt(d); invisible entries are *selected* to -inf (so whatever the
    hidden keys hold cannot reach the output); P = softmax(S); o = P v  -> [H, Lq, d].
    Reading: scale 1/sqrt(d), softmax in the working precision.
    """
    d = q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) * q.dtype.type(1.0 / math.sqrt(d))
    if visible is not None:
        s = np.where(visible[None, :, :], s, q.dtype.type(-np.inf))
    return softmax_rows(s) @ v


# ----------------------------------------------------------------------------------------------
# Time embedding and modulation ([ARCH] §2.3 input sequence: sinusoidal time embedding; single
# block: modulation of the normed input by shift/scale from the time embedding).
# ----------------------------------------------------------------------------------------------

def timestep_sinusoid(t: float, freq_dim: int, dt=np.float32) -> Array:
    """Sinusoidal embedding of the noise level s = 1000 (1 - t).

    Reading: t follows x_t = t x1 + (1-t) eps, and the pages' training pipeline samples a
    noise step in [0, 1000] with noise at the top, so the embedded scalar is s = 1000 (1 - t).
    emb = [cos(s w_i)]_i ++ [sin(s w_i)]_i with w_i = 10000^(-i/half), i < half = freq_dim/2.
    The angles and their cos/sin are evaluated in float64 and rounded once to the working type.
    """
    half = freq_dim // 2
    s = 1000.0 * (1.0 - float(t))
    omega = np.power(10000.0, -np.arange(half, dtype=np.float64) / half)
    arg = s * omega
    return np.concatenate([np.cos(arg), np.sin(arg)]).astype(dt)


def time_modulation(t: float, g: Dict[str, Array], freq_dim: int, dt=np.float32) -> Tuple[Array, Array]:
    """e = W2 SiLU(W1 emb + b1) + b2;  e6 = (Wp SiLU(e) + bp) as [6, D].

    Reading: one shared time projection to six vectors (shift1, scale1, gate1, shift2,
    scale2, gate2); each layer adds its own learned [6, D] offset.
    """
    emb = timestep_sinusoid(t, freq_dim, dt)
    e = linear(silu(linear(emb, g["t_w1"], g["t_b1"])), g["t_w2"], g["t_b2"])
    e6 = linear(silu(e), g["t_wp"], g["t_bp"])
    return e, e6.reshape(6, -1)


# ----------------------------------------------------------------------------------------------
# 3-D rotary embedding of video tokens ([ARCH] §2.3: video latents go through RoPE; action tokens
# do not). Reading: per-head channel pairs (2j, 2j+1); the first d_t/2 pairs rotate with the
# frame index, the next d_h/2 with the patch row, the last d_w/2 with the patch column;
# d_h = d_w = 2 floor(d/6), d_t = d - 2 d_h; frequency theta^(-2j'/d_axis) for local pair j'.
# ----------------------------------------------------------------------------------------------

def rope_axis_split(head_dim: int) -> Tuple[int, int, int]:
    dh = 2 * (head_dim // 6)
    return head_dim - 2 * dh, dh, dh


def rope_frequencies(head_dim: int, theta: float) -> Tuple[Array, Array]:
    """(axis index per pair in {0,1,2}, frequency per pair) for the head_dim/2 pairs."""
    dts = rope_axis_split(head_dim)
    axis, freq = [], []
    for a, da in enumerate(dts):
        for j in range(da // 2):
            axis.append(a)
            freq.append(theta ** (-2.0 * j / da))
    return np.array(axis, dtype=np.int64), np.array(freq, dtype=np.float64)


def video_positions(w, n_chunks: int, start_frame: int) -> Array:
    """(frame, row, col) of every video token of ``n_chunks`` consecutive chunks, [n*Lv, 3].

    Tokens of a chunk are in raster order (frame, row, col) (a reading of the pages); frame indices are
    absolute within the attention window: start_frame + chunk * frames_per_chunk + local frame
    ([WS1] continuous requests: the pipeline carries a frame position across requests).
    """
    Hp, Wp, Fc = w.grid_h, w.grid_w, w.frames_per_chunk
    out = []
    for c in range(n_chunks):
        for f in range(Fc):
            for r in range(Hp):
                for col in range(Wp):
                    out.append((start_frame + c * Fc + f, r, col))
    return np.array(out, dtype=np.int64)


def apply_rope(x: Array, pos: Array, head_dim: int, theta: float) -> Array:
    """Rotate x [T, H, d] (T tokens with positions pos [T, 3]) pair by pair.

    (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a), a = pos[axis(j)] * freq(j).
    Angles are formed in float64 and rounded once to the working precision.
    """
    axis, freq = rope_frequencies(head_dim, theta)
    ang = pos[:, axis].astype(np.float64) * freq[None, :]          # [T, d/2]
    c = np.cos(ang).astype(x.dtype)[:, None, :]
    s = np.sin(ang).astype(x.dtype)[:, None, :]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------------------------
# Model pieces
# ----------------------------------------------------------------------------------------------

def cast_params(p: Dict[str, Array], dt) -> Dict[str, Array]:
    return {k: np.asarray(v, dtype=dt) for k, v in p.items()}


def build_context(w, g: Dict[str, Array], txt: Array, img: Optional[Array], state: Optional[Array] = None) -> Array:
    """Condition sequence per CFG branch: [txt_b W_txt^T + b ; img W_img^T + b ; state W_st^T + b]
    -> [br, Lc, D].

    [ARCH] §2.1: image and text features (1536-d) are concatenated into one condition sequence;
    reading: one Linear per modality to the model width. Branch 1 carries the negative
    (null) prompt ([WS1] request format); the image features are shared by both branches.
    State rows: [HYPER] 方法 has proprioception pass a state encoder beside the text encoder
    before the modalities are fused into the causal DiT, and [N569] (architecture) counts that
    encoder among the few parameters added to the backbone. Here each proprioceptive feature
    vector [state_dim] goes through one Linear to one condition row after the image rows, shared
    by the branches; any featurisation of joint readings before it is the caller's.
    """
    ctx_t = linear(txt, g["txt_w"], g["txt_b"])                   # [br, Lt, D]
    parts = [ctx_t]
    br = ctx_t.shape[0]
    if img is not None and w.ctx_img_len > 0:
        ctx_i = linear(img, g["img_w"], g["img_b"])               # [Li, D]
        parts.append(np.broadcast_to(ctx_i[None], (br,) + ctx_i.shape))
    if getattr(w, "ctx_state_len", 0) > 0:
        assert state is not None and state.shape == (w.ctx_state_len, w.state_dim)
        ctx_s = linear(state, g["st_w"], g["st_b"])               # [Ls, D]
        parts.append(np.broadcast_to(ctx_s[None], (br,) + ctx_s.shape))
    return parts[0] if len(parts) == 1 else np.concatenate(parts, axis=1)


def context_kv(w, lp: Dict[str, Array], ctx: Array) -> Tuple[Array, Array]:
    """Per-layer cross-attention keys/values of the condition sequence (computed once per request:
    [ARCH] §4 encodes the conditions once and caches them). Kc = RMS(ctx Wck^T + b) g; Vc = ctx Wcv^T + b.
    Reading: RMSNorm on cross keys and queries, over the full width.
    """
    kc = rms_norm(linear(ctx, lp["w_ck"], lp["b_ck"]), w.eps, lp["g_ck"])
    vc = linear(ctx, lp["w_cv"], lp["b_cv"])
    if separate_image_attention(w):
        # image rows (after the text rows) through their own key / value projections and gain
        Lt = w.ctx_text_len
        kc = kc.copy()
        vc = vc.copy()
        kc[..., Lt:, :] = rms_norm(linear(ctx[..., Lt:, :], lp["w_cki"], lp["b_cki"]), w.eps, lp["g_cki"])
        vc[..., Lt:, :] = linear(ctx[..., Lt:, :], lp["w_cvi"], lp["b_cvi"])
    return kc, vc


def separate_image_attention(w) -> bool:
    """Variant drawn for the image-to-video backbone the architecture page builds on: the image part
    of the condition sequence has its own key / value projections and its own softmax, and the two
    attention outputs are summed before the output projection (bit 8 of ``variant``)."""
    return bool(getattr(w, "variant", 0) & 8)


def embed_tokens(g: Dict[str, Array], x_video: Array, x_action: Array, w, n_chunks: int) -> Array:
    """Token sequence of ``n_chunks`` chunks: per chunk [video rows ; action rows] -> [n*Lq, D].

    [ARCH] §2.3: video latent patches are projected and action tokens go through the action
    projection (one embodiment's Linear, [ARCH] §2.4), and both live in one sequence.
    x_video [n*Lv, P], x_action [n*La, A].
    """
    Lv, La = w.video_tokens, w.action_tokens
    hv = linear(x_video, g["pe_w"], g["pe_b"])
    ha = linear(x_action, g["ae_w"], g["ae_b"])
    rows = []
    for c in range(n_chunks):
        rows.append(hv[c * Lv:(c + 1) * Lv])
        rows.append(ha[c * La:(c + 1) * La])
    return np.concatenate(rows, axis=0)


def token_layout(w, n_chunks: int) -> Tuple[Array, Array, Array]:
    """(chunk index, group 0=video/1=action, index within the group of the chunk) per token."""
    Lv, La = w.video_tokens, w.action_tokens
    chunk, group, local = [], [], []
    for c in range(n_chunks):
        chunk += [c] * (Lv + La)
        group += [0] * Lv + [1] * La
        local += list(range(Lv)) + list(range(La))
    return np.array(chunk), np.array(group), np.array(local)


def feed_forward(w, lp: Dict[str, Array], y: Array) -> Array:
    """GELU_tanh(y W1^T + b1) W2^T + b2 (a reading of the pages); with the SwiGLU variant drawn on [ARCH] §2.3,
    (SiLU(y Wg^T + bg) * (y Wu^T + bu)) W2^T + b2 where rows 2j / 2j+1 of W1 (and entries of b1)
    are the gate / up rows of hidden unit j."""
    u = project(w, y, lp["w_ff1"], lp["b_ff1"])
    if getattr(w, "variant", 0) & 4:
        act = silu(u[..., 0::2]) * u[..., 1::2]
    else:
        act = gelu_tanh(u)
    return project(w, act, lp["w_ff2"], lp["b_ff2"])


def visibility(w, chunk: Array, group: Array, cached: int) -> Array:
    """[T, cached + T] mask of the self-attention (a reading of the pages): a query sees every cached clean key
    and the keys of earlier chunks of the pass; inside its own chunk it sees every token
    (bidirectional), or, with the frame-causal variant of [ARCH] §2.3 causal mask, a video token sees
    the video tokens of its own and earlier frames of the chunk and an action token the whole chunk."""
    T = chunk.size
    pos = np.zeros(T, dtype=np.int64)                  # index inside the chunk: video first, then actions
    for i in range(1, T):
        pos[i] = pos[i - 1] + 1 if chunk[i] == chunk[i - 1] else 0
    if getattr(w, "variant", 0) & 1:
        hw = w.grid_h * w.grid_w
        inside = np.where(group == 0, (pos // hw + 1) * hw, w.chunk_tokens)
    else:
        inside = np.full(T, w.chunk_tokens)
    same = chunk[None, :] == chunk[:, None]
    vis_pass = (chunk[None, :] < chunk[:, None]) | (same & (pos[None, :] < inside[:, None]))
    return np.concatenate([np.ones((T, cached), dtype=bool), vis_pass], axis=1)


@dataclass
class KVCache:
    """Per layer, per branch: keys (after RMSNorm and RoPE) and values of clean chunks.

    [WS1] architecture: the DiT runner maintains the attention KV; [HYPER] 方法: after a chunk
    executes, its entries are replaced by the encoding of the real observation.
    k[l], v[l]: [br, len, D].
    """
    k: List[Array] = field(default_factory=list)
    v: List[Array] = field(default_factory=list)

    @property
    def length(self) -> int:
        return 0 if not self.k else self.k[0].shape[1]

    @staticmethod
    def empty(layers: int, br: int, dim: int, dt=np.float32) -> "KVCache":
        z = np.zeros((br, 0, dim), dtype=dt)
        return KVCache([z.copy() for _ in range(layers)], [z.copy() for _ in range(layers)])


def block_forward(w, lp: Dict[str, Array], h: Array, mods: Array, ctx_k: Array, ctx_v: Array,
                  cache_k: Array, cache_v: Array, n_chunks: int, pos: Array) -> Tuple[Array, Array, Array]:
    """One causal DiT block on all CFG branches.

    h [br, T, D] (T = n_chunks * Lq), mods [T, 6, D] = per-token time modulation (e6 of the token's
    chunk and group; the layer offset is added here), ctx_k/ctx_v [br, Lc, D], cache_k/cache_v
    [br, len, D] (clean chunks before these), pos [n*Lv, 3] video positions.
    Returns (h_out, k_new, v_new) where k_new/v_new [br, T, D] are this call's keys/values.

    Order ([ARCH] §2.3 single block): norm -> modulation -> causal self-attention -> residual ->
    norm -> cross-attention -> residual -> norm -> FFN -> residual. Readings: gates on the
    self-attention and FFN residuals only, scale entering as (1 + scale); LayerNorm; GELU-tanh FFN;
    chunk-level mask, bidirectional inside a chunk; RoPE as in apply_rope; cross q/k RMSNorm.
    """
    br, T, D = h.shape
    H, d = w.heads, w.head_dim
    dt = h.dtype
    m = mods + lp["mod"][None, :, :]                              # [T, 6, D]
    shift1, scale1, gate1, shift2, scale2, gate2 = (m[:, i, :] for i in range(6))
    chunk, group, _ = token_layout(w, n_chunks)
    is_video = group == 0
    L0 = cache_k.shape[1]
    visible = visibility(w, chunk, group, L0)
    oc_all = np.empty_like(h)
    k_new = np.empty_like(h)
    v_new = np.empty_like(h)
    # --- self-attention sub-layer
    o_all = np.empty_like(h)
    for b in range(br):
        y = modulated_norm(h[b], shift1, scale1, w.eps, uses_rms(w))
        qkv = project(w, y, lp["w_qkv"], lp["b_qkv"])
        q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
        q = rms_norm(q, w.eps, lp["g_q"]).reshape(T, H, d)
        k = rms_norm(k, w.eps, lp["g_k"]).reshape(T, H, d)
        q[is_video] = apply_rope(q[is_video], pos, d, w.rope_theta)
        k[is_video] = apply_rope(k[is_video], pos, d, w.rope_theta)
        k_new[b] = k.reshape(T, D)
        v_new[b] = v
        kk = np.concatenate([cache_k[b], k_new[b]], axis=0).reshape(-1, H, d).transpose(1, 0, 2)
        vv = np.concatenate([cache_v[b], v_new[b]], axis=0).reshape(-1, H, d).transpose(1, 0, 2)
        o = attention(q.transpose(1, 0, 2), kk, vv, visible)      # [H, T, d]
        o_all[b] = o.transpose(1, 0, 2).reshape(T, D)
    h = h + gate1[None] * project(w, o_all, lp["w_o"], lp["b_o"])
    # --- cross-attention sub-layer (no mask, no RoPE, no modulation)
    for b in range(br):
        n3 = (rms_norm(h[b], w.eps) * lp["ln3_w"] + lp["ln3_b"] if uses_rms(w)
              else layer_norm(h[b], w.eps, lp["ln3_w"], lp["ln3_b"]))
        qc = rms_norm(project(w, n3, lp["w_cq"], lp["b_cq"]), w.eps, lp["g_cq"]).reshape(T, H, d)
        kc = ctx_k[b].reshape(-1, H, d).transpose(1, 0, 2)
        vc = ctx_v[b].reshape(-1, H, d).transpose(1, 0, 2)
        if separate_image_attention(w):
            Lt = w.ctx_text_len
            oc = (attention(qc.transpose(1, 0, 2), kc[:, :Lt], vc[:, :Lt], None)
                  + attention(qc.transpose(1, 0, 2), kc[:, Lt:], vc[:, Lt:], None))
            oc = oc.transpose(1, 0, 2).reshape(T, D)
        else:
            oc = attention(qc.transpose(1, 0, 2), kc, vc, None).transpose(1, 0, 2).reshape(T, D)
        oc_all[b] = oc
    h = h + project(w, oc_all, lp["w_co"], lp["b_co"])
    # --- feed-forward sub-layer
    y2 = modulated_norm(h, shift2[None], scale2[None], w.eps, uses_rms(w))
    h = h + gate2[None] * feed_forward(w, lp, y2)
    return h, k_new, v_new


def per_token_time(w, g: Dict[str, Array], t_video: Sequence[float], t_action: Sequence[float],
                   n_chunks: int, dt) -> Tuple[Array, Array]:
    """Per-token e6 [T, 6, D] and e [T, D]: the token's chunk picks its timesteps and its group
    (video/action) picks t_video or t_action ([N569] DreamZero-Flash: decoupled video and action
    noise levels; with equal values this is the shared timestep of the standard model)."""
    chunk, group, _ = token_layout(w, n_chunks)
    table_e6, table_e = {}, {}
    for c in range(n_chunks):
        for gi, t in ((0, t_video[c]), (1, t_action[c])):
            table_e[(c, gi)], table_e6[(c, gi)] = time_modulation(t, g, w.freq_dim, dt)
    e6 = np.stack([table_e6[(c, gi)] for c, gi in zip(chunk, group)])
    e = np.stack([table_e[(c, gi)] for c, gi in zip(chunk, group)])
    return e6, e


def embodiment_params(g: Dict[str, Array], e: int) -> Dict[str, Array]:
    """Global parameters routed to embodiment e ([ARCH] §2.4: each robot body has its own action
    encoder and decoder linear around the shared DiT, chosen by the embodiment id): ae_* / ao_* are
    replaced by that embodiment's (embodiment 0 keeps the defaults); everything else is shared."""
    if e == 0:
        return g
    out = dict(g)
    for name in ("ae_w", "ae_b", "ao_w", "ao_b"):
        out[name] = g["%s_%d" % (name, e)]
    return out


def head_forward(w, g: Dict[str, Array], h: Array, e: Array, n_chunks: int) -> Tuple[Array, Array]:
    """Output split ([ARCH] §2.3 output decoding, §2.4 per-embodiment decoder):
    n = LN(h)(1 + scale_h) + shift_h with (shift_h, scale_h) = head_mod + e;
    v_video = n_video W_vo^T + b, v_action = n_action W_ao^T + b."""
    shift = g["head_mod"][0][None] + e
    scale = g["head_mod"][1][None] + e
    n = modulated_norm(h, shift[None], scale[None], w.eps, uses_rms(w))
    _, group, _ = token_layout(w, n_chunks)
    vv = linear(n[:, group == 0], g["vo_w"], g["vo_b"])
    va = linear(n[:, group == 1], g["ao_w"], g["ao_b"])
    return vv, va


@dataclass
class Model:
    """Weights of the stack as float arrays: ``g`` global, ``layers[l]`` per layer."""
    w: object
    g: Dict[str, Array]
    layers: List[Dict[str, Array]]


def stack_forward(model: Model, cache: KVCache, ctx_kv: List[Tuple[Array, Array]],
                  x_video: Array, x_action: Array, t_video: Sequence[float], t_action: Sequence[float],
                  n_chunks: int, start_frame: int, dt=np.float32, commit: bool = False,
                  layer_fn=None) -> Tuple[Array, Array]:
    """One pass of the DiT over ``n_chunks`` chunks on all CFG branches.

    x_video [n*Lv, P], x_action [n*La, A] (the same noisy latents for every branch);
    returns per-branch velocities (v_video [br, n*Lv, P], v_action [br, n*La, A]).
    With n_chunks = 1 and a cache of clean chunks this is the incremental step; with n_chunks > 1
    it is the full-sequence pass under the chunk-causal mask ([HYPER] 方法, teacher forcing).
    commit=True appends this call's keys/values to ``cache`` ([N569] inference: KV cache with
    real observations).
    """
    w = model.w
    g = model.g
    br = w.branches
    e6, e = per_token_time(w, g, t_video, t_action, n_chunks, dt)
    h0 = embed_tokens(g, x_video.astype(dt), x_action.astype(dt), w, n_chunks)
    h = np.broadcast_to(h0[None], (br,) + h0.shape).astype(dt).copy()
    pos = video_positions(w, n_chunks, start_frame)
    new_k, new_v = [], []
    for l, lp in enumerate(model.layers):
        ck, cv = ctx_kv[l]
        if cache.k:
            kc, vc = cache.k[l].astype(dt), cache.v[l].astype(dt)
        else:
            kc = vc = np.zeros((br, 0, w.dim), dtype=dt)
        h, kn, vn = (layer_fn or block_forward)(w, lp, h, e6, ck, cv, kc, vc, n_chunks, pos)
        new_k.append(kn)
        new_v.append(vn)
    if commit:
        for l in range(len(model.layers)):
            cache.k[l] = np.concatenate([cache.k[l].astype(dt), new_k[l]], axis=1)
            cache.v[l] = np.concatenate([cache.v[l].astype(dt), new_v[l]], axis=1)
    return head_forward(w, g, h, e, n_chunks)


@dataclass
class PassSpec:
    """One stack pass for ``stack_passes``: its chunks' latents and timesteps as for stack_forward,
    whether it commits its keys/values, and whether its head outputs are wanted."""
    x_video: Array
    x_action: Array
    t_video: Sequence[float]
    t_action: Sequence[float]
    n_chunks: int
    start_frame: int
    commit: bool = False
    heads: bool = True


def stack_passes(model: Model, ctx: Array, passes: Sequence[PassSpec], dt=np.float32,
                 cache: Optional[KVCache] = None, progress=None) -> List[Optional[Tuple[Array, Array]]]:
    """Several stack passes in the given order, each seeing the KV cache as the earlier passes left
    it: the result equals calling stack_forward for each pass in turn (commit appends a pass's
    keys/values, kv_append is a committing pass at t = 1 without heads). A pass's block l depends on
    the earlier passes only through their layer-l keys/values, so the passes advance together layer
    by layer: each layer's weights (``model.layers[l]``, which may be drawn on demand) and its
    condition keys/values (from ``ctx`` [br, Lc, D], as context_kv) are formed once and dropped after
    use. ``cache`` (default: empty) is extended in place. Returns per pass (v_video, v_action), or
    None where heads=False. ``progress(l)`` is called after each layer."""
    w, g = model.w, model.g
    br = w.branches
    L = len(model.layers)
    if cache is None:
        cache = KVCache.empty(L, br, w.dim, dt)
    states = []
    for p in passes:
        e6, e = per_token_time(w, g, p.t_video, p.t_action, p.n_chunks, dt)
        h0 = embed_tokens(g, p.x_video.astype(dt), p.x_action.astype(dt), w, p.n_chunks)
        h = np.broadcast_to(h0[None], (br,) + h0.shape).astype(dt).copy()
        states.append([h, e6, e, video_positions(w, p.n_chunks, p.start_frame)])
    for l in range(L):
        lp = model.layers[l]
        ck, cv = context_kv(w, lp, ctx)
        kc, vc = cache.k[l].astype(dt), cache.v[l].astype(dt)
        for st, p in zip(states, passes):
            st[0], kn, vn = block_forward(w, lp, st[0], st[1], ck, cv, kc, vc, p.n_chunks, st[3])
            if p.commit:
                kc = np.concatenate([kc, kn], axis=1)
                vc = np.concatenate([vc, vn], axis=1)
        cache.k[l], cache.v[l] = kc, vc
        del lp, ck, cv
        if progress is not None:
            progress(l)
    return [head_forward(w, g, st[0], st[2], p.n_chunks) if p.heads else None for st, p in zip(states, passes)]


def kv_append(model: Model, cache: KVCache, ctx_kv, x_video: Array, x_action: Array,
              start_frame: int, dt=np.float32) -> None:
    """Commit one clean chunk: a stack pass at t_video = t_action = 1 whose keys/values are
    appended (reading: cached chunks are clean, t = 1). [HYPER] 方法: predicted frames in the
    KV cache are replaced by real observations after the chunk executes."""
    stack_forward(model, cache, ctx_kv, x_video, x_action, [1.0], [1.0], 1, start_frame, dt, commit=True)


def kv_evict(w, cache: KVCache, drop_rows: int, frame_shift: int) -> None:
    """Slide the attention window ([WS1] continuous requests: the window releases old KV and the
    frame position restarts): drop the oldest ``drop_rows`` cached rows (whole chunks) and move the
    kept chunks' frame positions back by ``frame_shift``. Cached keys are stored after RoPE, so the
    video keys are rotated once more with position (-frame_shift, 0, 0): the frame-axis pairs turn
    by -frame_shift * freq, the row and column pairs by zero. Values and action keys only move."""
    Lq, Lv = w.chunk_tokens, w.video_tokens
    assert 0 <= drop_rows <= cache.length and drop_rows % Lq == 0
    keep = cache.length - drop_rows
    is_video = (np.arange(keep) % Lq) < Lv
    H, d = w.heads, w.head_dim
    pos = np.tile(np.array([[-frame_shift, 0, 0]], dtype=np.int64), (int(is_video.sum()), 1))
    for l in range(len(cache.k)):
        k = cache.k[l][:, drop_rows:].copy()
        for b in range(k.shape[0]):
            kb = k[b].reshape(keep, H, d)
            kb[is_video] = apply_rope(kb[is_video], pos, d, w.rope_theta)
            k[b] = kb.reshape(keep, H * d)
        cache.k[l] = k
        cache.v[l] = cache.v[l][:, drop_rows:].copy()


# ----------------------------------------------------------------------------------------------
# Guidance, Euler update, velocity reuse ([N569] real-time optimisations; Euler on the step grid)
# ----------------------------------------------------------------------------------------------

def cfg_combine(v_branches: Array, guidance: float) -> Array:
    """Classifier-free guidance: v = v_uncond + w (v_cond - v_uncond); branch 0 is conditional,
    branch 1 the negative/null prompt ([N569]: the conditional and unconditional passes; [WS1]
    request format: negative prompt). Reading: w applies to video and action alike; the sum
    is evaluated as w v_cond + (1 - w) v_uncond, which is the same quantity and returns either
    branch exactly at w = 1 or w = 0."""
    v0, v1 = v_branches[0], v_branches[1]
    wc = v_branches.dtype.type(guidance)
    wu = v_branches.dtype.type(1.0 - guidance)
    return wc * v0 + wu * v1


def euler_update(x: Array, v: Array, t: float, t_next: float) -> Array:
    """x <- x + (t_next - t) v (reading: Euler on the flow-matching ODE)."""
    return x + x.dtype.type(t_next - t) * v


def interpolate(x1: Array, eps: Array, t: float) -> Array:
    """x_t = t x1 + (1 - t) eps (reading of the pages' linear interpolation)."""
    return x1.dtype.type(t) * x1 + x1.dtype.type(1.0 - t) * eps


def cosine_fp64(a: Array, b: Array) -> float:
    """Cosine similarity of two flattened tensors, accumulated in float64."""
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / math.sqrt((a @ a) * (b @ b)))


def denoise_chunk(dit, x_video: Array, x_action: Array, grid: Sequence[float], tau: float,
                  max_consecutive_reuse: Optional[int] = None, trace: Optional[list] = None):
    """Euler loop with velocity reuse ([N569] DiT caching; [WS1] dynamic16).

    dit(x_video, x_action, t) -> guided (v_video, v_action). Steps 0 and 1 always run the DiT;
    at step k >= 2, if the cosine similarity of the two most recent DiT-computed guided video
    velocities exceeds tau, the DiT is skipped and the latest computed velocity is reused
    (a reading of the pages). Returns (x_video, x_action, number of DiT calls, per-step flags). ``trace``, if
    given, receives (k, cosine) for every step whose decision evaluated a cosine.
    """
    computed: List[Tuple[Array, Array]] = []
    calls = 0
    consecutive = 0
    flags = []
    xv, xa = x_video.copy(), x_action.copy()
    for k in range(len(grid) - 1):
        t, tn = grid[k], grid[k + 1]
        reuse = False
        if k >= 2 and len(computed) >= 2:
            c = cosine_fp64(computed[-1][0], computed[-2][0])
            if trace is not None:
                trace.append((k, c))
            if c > tau and (max_consecutive_reuse is None or consecutive < max_consecutive_reuse):
                reuse = True
        if reuse:
            vv, va = computed[-1]
            consecutive += 1
        else:
            vv, va = dit(xv, xa, t)
            computed.append((vv, va))
            calls += 1
            consecutive = 0
        flags.append(reuse)
        xv = euler_update(xv, vv, t, tn)
        xa = euler_update(xa, va, t, tn)
    return xv, xa, calls, flags


# ----------------------------------------------------------------------------------------------
# Loading the synthetic weights as float arrays
# ----------------------------------------------------------------------------------------------

class LazyLayers:
    """The per-layer weights of a workload, drawn from ``synth`` each time a layer is asked for and
    not kept: a 40-layer model in float32 is 57 GB, one layer 1.4 GB."""

    def __init__(self, w, dt=np.float32):
        self.w, self.dt = w, dt

    def __len__(self) -> int:
        return self.w.layers

    def __getitem__(self, l: int) -> Dict[str, Array]:
        from synth.workloads import draw, layer_tensors
        if not 0 <= l < self.w.layers:
            raise IndexError(l)
        return {s[0]: draw(self.w, l, s, "f32").astype(self.dt) for s in layer_tensors(self.w)}

    def __iter__(self):
        return (self[l] for l in range(len(self)))


def load_model_lazy(w, dt=np.float32) -> Model:
    """As load_model, with the layers drawn on demand (LazyLayers)."""
    from synth.workloads import draw, global_tensors
    g = {s[0]: draw(w, -1, s, "f32").astype(dt) for s in global_tensors(w)}
    return Model(w, g, LazyLayers(w, dt))


def load_model(w, dt=np.float32, layers: Optional[Sequence[int]] = None) -> Model:
    """Draw the workload's weights (bf16-representable values) from ``synth`` as ``dt`` arrays."""
    import synth
    from synth.workloads import draw, global_tensors, layer_tensors
    g = {s[0]: draw(w, -1, s, "f32").astype(dt) for s in global_tensors(w)}
    ls = range(w.layers) if layers is None else layers
    lay = [{s[0]: draw(w, l, s, "f32").astype(dt) for s in layer_tensors(w)} for l in ls]
    return Model(w, g, lay)
