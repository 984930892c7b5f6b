"""Synthetic workload recipes: sizes, tensor names, shapes and value distributions.

Shapes follow the pages: Wan2.1-14B backbone sizes (40 layers, width 5120,
40 heads of 128, FFN 13824; DreamZero architecture page, hyper-parameter
table), 320x176 frames -> 40x22 latents -> 2x2 patches of 16 channels (VAE
section), a 24-step action horizon with DROID's 8-d actions (PhyAI ws1 page,
request format), 512 text tokens and 1536-d encoder features (same pages),
three stitched camera views (paper walk-through, architecture). Weights are
N(0, 0.02), norm gains 1 and LayerNorm biases 0, condition features and noise
N(0, 1), clean actions U(-1, 1).

This file contains no arithmetic of the method; it only says what to draw.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    id: int
    name: str
    dim: int
    heads: int
    head_dim: int
    ffn_dim: int
    layers: int
    freq_dim: int = 256
    patch_dim: int = 64
    action_dim: int = 8
    action_tokens: int = 24
    frames_per_chunk: int = 2
    grid_h: int = 11
    grid_w: int = 20
    ctx_in_dim: int = 1536
    ctx_text_len: int = 512
    ctx_img_len: int = 257
    branches: int = 2
    cache_chunks: int = 1
    eps: float = 1e-6
    rope_theta: float = 10000.0
    guidance: float = 5.0
    variant: int = 0        # architectural variants of the pages (bit flags, see VARIANT_* below)
    precision: int = 0      # arithmetic of the block projections: 0 the model dtype, PRECISION_MXFP8
    embodiments: int = 1    # action encoder / decoder pairs; embodiment 0 is ae_* / ao_*, e >= 1 ae_*_e / ao_*_e
    ctx_state_len: int = 0  # proprioceptive state rows appended to the condition sequence (0: none)
    state_dim: int = 64     # width of one (normalised, padded) state vector

    @property
    def video_tokens(self) -> int:
        return self.frames_per_chunk * self.grid_h * self.grid_w

    @property
    def chunk_tokens(self) -> int:
        return self.video_tokens + self.action_tokens

    @property
    def ctx_len(self) -> int:
        return self.ctx_text_len + self.ctx_img_len + self.ctx_state_len

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# Variants drawn on the architecture page next to the adopted readings (bit flags):
VARIANT_FRAME_CAUSAL = 1   # inside a chunk a frame sees earlier and its own frames; actions see the chunk
VARIANT_RMS_NORM = 2       # RMSNorm in place of the block and head LayerNorms
VARIANT_SWIGLU = 4         # SwiGLU feed-forward: SiLU(gate) * up with interleaved [gate, up] rows
VARIANT_IMG_XATTN = 8      # image condition tokens: own key / value projections and their own softmax

# Low-precision block projections: inputs and weights quantised to MXFP8 (fp8 e4m3 codes with one
# power-of-two scale per 32 consecutive input features)
PRECISION_MXFP8 = 1
PRECISION_MXFP4W = 2       # weights MXFP4 (fp4 e2m1 codes, same block scales), activations MXFP8

WORKLOADS = {
    # Tiny single block: width 256, 4 heads of 64, FFN 1024, 2 frames of 8x8 patches + 24 action tokens,
    # 32 text tokens of width 256 and no image tokens; chunk 0 clean in the cache, chunk 1 noisy at t=0.5.
    1: Workload(1, "tiny-block-f32", dim=256, heads=4, head_dim=64, ffn_dim=1024, layers=1,
                grid_h=8, grid_w=8, ctx_in_dim=256, ctx_text_len=32, ctx_img_len=0, cache_chunks=1),
    # One full-width block (bf16), one clean chunk cached.
    2: Workload(2, "wan14b-block-bf16", dim=5120, heads=40, head_dim=128, ffn_dim=13824, layers=1,
                cache_chunks=1),
    # Full 40-layer step, CFG as batch 2, two clean chunks cached (928 rows).
    3: Workload(3, "wan14b-40L-cfg2-step-bf16", dim=5120, heads=40, head_dim=128, ffn_dim=13824, layers=40,
                cache_chunks=2),
    # Four successive chunks of 16 Euler steps each, starting from one cached chunk.
    4: Workload(4, "wan14b-40L-4chunk-16step-bf16", dim=5120, heads=40, head_dim=128, ffn_dim=13824,
                layers=40, cache_chunks=1),
    # Three stitched views (120x22 patches per frame -> 660 tokens), six clean chunks cached (8064 rows).
    5: Workload(5, "wan14b-40L-3view-longctx-bf16", dim=5120, heads=40, head_dim=128, ffn_dim=13824,
                layers=40, grid_h=11, grid_w=60, cache_chunks=6),
}


def global_tensors(w: Workload):
    """(name, shape, kind, sigma_or_value) of the tensors shared by all layers."""
    D, P, A, C = w.dim, w.patch_dim, w.action_dim, w.ctx_in_dim
    out = [
        ("t_w1", (D, w.freq_dim), "normal", 0.02), ("t_b1", (D,), "normal", 0.02),
        ("t_w2", (D, D), "normal", 0.02), ("t_b2", (D,), "normal", 0.02),
        ("t_wp", (6 * D, D), "normal", 0.02), ("t_bp", (6 * D,), "normal", 0.02),
        ("pe_w", (D, P), "normal", 0.02), ("pe_b", (D,), "normal", 0.02),
        ("ae_w", (D, A), "normal", 0.02), ("ae_b", (D,), "normal", 0.02),
        ("txt_w", (D, C), "normal", 0.02), ("txt_b", (D,), "normal", 0.02),
        ("head_mod", (2, D), "normal", 0.02),
        ("vo_w", (P, D), "normal", 0.02), ("vo_b", (P,), "normal", 0.02),
        ("ao_w", (A, D), "normal", 0.02), ("ao_b", (A,), "normal", 0.02),
    ]
    if w.ctx_img_len > 0:
        out += [("img_w", (D, C), "normal", 0.02), ("img_b", (D,), "normal", 0.02)]
    if w.ctx_state_len > 0:
        out += [("st_w", (D, w.state_dim), "normal", 0.02), ("st_b", (D,), "normal", 0.02)]
    for e in range(1, w.embodiments):
        out += [("ae_w_%d" % e, (D, A), "normal", 0.02), ("ae_b_%d" % e, (D,), "normal", 0.02),
                ("ao_w_%d" % e, (A, D), "normal", 0.02), ("ao_b_%d" % e, (A,), "normal", 0.02)]
    return out


def layer_tensors(w: Workload):
    """(name, shape, kind, sigma_or_value) of one layer's tensors (Linear weights are [out, in])."""
    D, F = w.dim, w.ffn_dim
    F1 = 2 * F if w.variant & VARIANT_SWIGLU else F   # SwiGLU: interleaved gate and up rows
    n = lambda name, shape: (name, shape, "normal", 0.02)  # noqa: E731
    c = lambda name, shape, v: (name, shape, "const", v)  # noqa: E731
    return [
        n("mod", (6, D)),
        n("w_qkv", (3 * D, D)), n("b_qkv", (3 * D,)), c("g_q", (D,), 1.0), c("g_k", (D,), 1.0),
        n("w_o", (D, D)), n("b_o", (D,)),
        c("ln3_w", (D,), 1.0), c("ln3_b", (D,), 0.0),
        n("w_cq", (D, D)), n("b_cq", (D,)), c("g_cq", (D,), 1.0),
        n("w_ck", (D, D)), n("b_ck", (D,)), c("g_ck", (D,), 1.0),
        n("w_cv", (D, D)), n("b_cv", (D,)),
        n("w_co", (D, D)), n("b_co", (D,)),
        n("w_ff1", (F1, D)), n("b_ff1", (F1,)),
        n("w_ff2", (D, F)), n("b_ff2", (D,)),
    ] + ([n("w_cki", (D, D)), n("b_cki", (D,)), c("g_cki", (D,), 1.0), n("w_cvi", (D, D)), n("b_cvi", (D,))]
         if w.variant & VARIANT_IMG_XATTN else [])


def input_tensors(w: Workload, n_chunks: int):
    """Condition features and, per chunk c, clean data and noise for video and action."""
    out = [("txt", (w.branches, w.ctx_text_len, w.ctx_in_dim), "normal", 1.0)]
    if w.ctx_img_len > 0:
        out.append(("img", (w.ctx_img_len, w.ctx_in_dim), "normal", 1.0))
    for c in range(n_chunks if w.ctx_state_len > 0 else 0):   # the observed state of each chunk
        out.append(("state_%d" % c, (w.ctx_state_len, w.state_dim), "normal", 1.0))
    for c in range(n_chunks):
        out += [
            ("x1_video_%d" % c, (w.video_tokens, w.patch_dim), "normal", 1.0),
            ("eps_video_%d" % c, (w.video_tokens, w.patch_dim), "normal", 1.0),
            ("x1_action_%d" % c, (w.action_tokens, w.action_dim), "uniform", None),
            ("eps_action_%d" % c, (w.action_tokens, w.action_dim), "normal", 1.0),
        ]
    return out


MATRIX_NAMES = frozenset({
    "t_w1", "t_w2", "t_wp", "pe_w", "ae_w", "txt_w", "img_w", "vo_w", "ao_w", "st_w",
    "w_qkv", "w_o", "w_cq", "w_ck", "w_cv", "w_co", "w_ff1", "w_ff2", "w_cki", "w_cvi",
})


def is_matrix(name: str) -> bool:
    """Linear weights ([out, in]) are the tensors a bf16 path stores in bf16; every other tensor
    (biases, gains, LayerNorm affine vectors, modulation tables) stays float32."""
    return name in MATRIX_NAMES or name.rsplit("_", 1)[0] in ("ae_w", "ao_w")


def draw(w: Workload, layer: int, spec, fmt: str = "f32"):
    """Materialise one (name, shape, kind, arg) spec for ``layer`` (-1 = global / inputs)."""
    from . import constant, fill, tensor_key
    name, shape, kind, arg = spec
    if kind == "const":
        return constant(shape, arg, fmt)
    key = tensor_key(w.id, layer, name)
    if kind == "normal":
        return fill(shape, key, "normal", sigma=arg, fmt=fmt)
    return fill(shape, key, "uniform", fmt=fmt)


def draw_named(w: Workload, layer: int, name: str, fmt: str = "f32", n_chunks: int = 8):
    specs = {s[0]: s for s in (layer_tensors(w) if layer >= 0 else global_tensors(w) + input_tensors(w, n_chunks))}
    return draw(w, layer, specs[name], fmt)


def timesteps(w: Workload, n: int, stream: int = 1) -> np.ndarray:
    """n scalars U(0, 1) from the workload's timestep stream (host floats)."""
    from . import tensor_key, uniform01
    return uniform01(n, tensor_key(w.id, -1, "timesteps"), stream=stream)
