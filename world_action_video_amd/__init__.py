"""Python binding of ``libwam.so``: the C-ABI calls under the same names, argument marshalling only.

Every step of the denoising path runs in the library's HIP kernels; this module only converts
Python objects (torch tensors, ints, floats) into the C structs and pointers of ``include/wam.h``.
Importing works without a GPU; calling anything needs the built library (``build.build()``) and
raises if it is missing -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwam.so")

WAM_OK, WAM_E_ARG, WAM_E_SHAPE, WAM_E_CAPACITY, WAM_E_HIP, WAM_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
WAM_BF16, WAM_F32 = 0, 1
WAM_PRECISION_NATIVE, WAM_PRECISION_MXFP8, WAM_PRECISION_MXFP4W = 0, 1, 2
WAM_MX_E4M3, WAM_MX_E2M1 = 0, 1

EXPORTS = ("wam_workspace_bytes", "wam_ctx_build", "wam_ctx_set_state", "wam_time_embed", "wam_dit_stack_fwd", "wam_kv_append",
           "wam_dit_block_fwd", "wam_flow_step", "wam_denoise_chunk", "wam_denoise_chunk_unipc", "wam_op_linear",
           "wam_mx_quantize", "wam_mx4_quantize", "wam_op_linear_mx", "wam_mx_block_bytes", "wam_mx_pack_block",
           "wam_weights_for_embodiment", "wam_op_attention", "wam_kv_evict", "wam_kv_reset", "wam_last_error",
           "wam_qkv_timer_config", "wam_qkv_timer_read", "wam_op_attention_mx", "wam_flow_step_noalloc",
           "wam_denoise_chunk_replay", "wam_mfma_peak_probe", "wam_op_split_finish", "wam_op_modulated_norm",
           "wam_op_qkv_cache", "wam_pack_weight", "wam_op_linear_packed", "wam_pack_block_bytes", "wam_pack_block")


class WamError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("wam status %d: %s" % (status, msg))
        self.status = status


class wam_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("dim", "heads", "head_dim", "ffn_dim", "layers", "freq_dim",
                                             "patch_dim", "action_dim", "action_tokens", "frames_per_chunk",
                                             "grid_h", "grid_w", "ctx_in_dim", "ctx_text_len", "ctx_img_len",
                                             "branches")] + \
              [("rope_theta", ctypes.c_float), ("eps", ctypes.c_float), ("dtype", ctypes.c_int),
               ("variant", ctypes.c_int), ("precision", ctypes.c_int), ("ctx_state_len", ctypes.c_int),
               ("state_dim", ctypes.c_int)]


BLOCK_FIELDS = ("mod", "w_qkv", "b_qkv", "g_q", "g_k", "w_o", "b_o", "ln3_w", "ln3_b", "w_cq", "b_cq", "g_cq",
                "w_ck", "b_ck", "g_ck", "w_cv", "b_cv", "w_co", "b_co", "w_ff1", "b_ff1", "w_ff2", "b_ff2")
IMG_XATTN_FIELDS = ("w_cki", "b_cki", "g_cki", "w_cvi", "b_cvi")
GLOBAL_FIELDS = ("t_w1", "t_b1", "t_w2", "t_b2", "t_wp", "t_bp", "pe_w", "pe_b", "ae_w", "ae_b", "head_mod",
                 "vo_w", "vo_b", "ao_w", "ao_b", "txt_w", "txt_b", "img_w", "img_b")


class wam_block_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_FIELDS] + [("mx", ctypes.c_void_p)] + \
               [(n, ctypes.c_void_p) for n in IMG_XATTN_FIELDS] + [("pk", ctypes.c_void_p)]


class wam_action_io(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ae_w", "ae_b", "ao_w", "ao_b")]


class wam_weights(ctypes.Structure):
    _fields_ = [("blocks", ctypes.POINTER(wam_block_weights))] + [(n, ctypes.c_void_p) for n in GLOBAL_FIELDS] + \
               [("embodiments", ctypes.POINTER(wam_action_io)), ("n_embodiments", ctypes.c_int),
                ("st_w", ctypes.c_void_p), ("st_b", ctypes.c_void_p)]


class wam_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("branches", ctypes.c_int),
                ("capacity", ctypes.c_int), ("length", ctypes.c_int)]


class wam_ctx_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("branches", ctypes.c_int),
                ("ctx_len", ctypes.c_int), ("ctx_stride", ctypes.c_int)]


_lib = None


def load(path: str = LIB_PATH):
    """Load ``libwam.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libwam.so is not built (run world_action_video_amd/build.py); no fallback exists")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    CFG = ctypes.POINTER(wam_config)
    W = ctypes.POINTER(wam_weights)
    KV = ctypes.POINTER(wam_kv_cache)
    CX = ctypes.POINTER(wam_ctx_kv)
    sig = {
        "wam_workspace_bytes": (S, [CFG, I]),
        "wam_ctx_build": (I, [CFG, W, P, P, P, CX, P, S, P]),
        "wam_ctx_set_state": (I, [CFG, W, P, CX, P, S, P]),
        "wam_time_embed": (I, [CFG, W, P, I, P, P, P, S, P]),
        "wam_dit_stack_fwd": (I, [CFG, W, KV, CX, I, P, P, P, P, I, P, P, P, S, P]),
        "wam_kv_append": (I, [CFG, W, KV, CX, P, P, I, P, S, P]),
        "wam_dit_block_fwd": (I, [CFG, ctypes.POINTER(wam_block_weights), I, KV, CX, P, P, I, I, I, P, S, P]),
        "wam_flow_step": (I, [P, P, P, P, I, F, I, I, F, F, P, P, P, P, P, S, P]),
        "wam_flow_step_noalloc": (I, [P, P, P, P, I, F, I, I, F, F, P, P, P, P, P]),
        "wam_denoise_chunk": (I, [CFG, W, KV, CX, P, P, P, I, F, F, I, I, P, P, P, P, P, P, S, P, P, P]),
        "wam_denoise_chunk_replay": (I, [CFG, W, KV, CX, P, P, P, I, F, P, I, P, P, P, P, P, P, S, P, P, P]),
        "wam_denoise_chunk_unipc": (I, [CFG, W, KV, CX, P, P, P, I, F, F, I, I, I, I, P, P, P, P, P, P, P, S, P, P,
                                        P]),
        "wam_op_linear": (I, [I, P, I, P, I, P, P, I, I, I, I, I, P, S, P]),
        "wam_mx_quantize": (I, [I, P, I, I, I, P, I, P, P]),
        "wam_mx4_quantize": (I, [I, P, I, I, I, P, I, P, P]),
        "wam_mx_block_bytes": (S, [CFG]),
        "wam_weights_for_embodiment": (I, [ctypes.POINTER(wam_weights), I, ctypes.POINTER(wam_weights)]),
        "wam_mx_pack_block": (I, [CFG, ctypes.POINTER(wam_block_weights), P, S, P]),
        "wam_op_linear_mx": (I, [P, P, I, P, P, I, I, P, P, I, I, I, I, I, P, S, P]),
        "wam_op_attention": (I, [I, P, P, P, P, I, I, I, I, I, I, I, I, I, P, S, P]),
        "wam_kv_evict": (I, [CFG, KV, I, I, P]),
        "wam_kv_reset": (None, [KV]),
        "wam_last_error": (ctypes.c_char_p, []),
        "wam_qkv_timer_config": (I, [I, I]),
        "wam_qkv_timer_read": (I, [ctypes.POINTER(ctypes.c_float), I, ctypes.POINTER(ctypes.c_int)]),
        "wam_op_attention_mx": (I, [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]),
        "wam_mfma_peak_probe": (I, [P, I, I, P]),
        "wam_op_split_finish": (I, [P, I, I, I, P, P, P, P, I, P, I, I, I, F, P, P]),
        "wam_op_modulated_norm": (I, [P, I, I, P, P, I, I, I, F, P, P]),
        "wam_op_qkv_cache": (I, [P, I, I, I, I, I, I, P, P, F, P, P, P, P, I, I, P]),
        "wam_pack_weight": (I, [P, I, I, I, P, P]),
        "wam_op_linear_packed": (I, [P, I, P, P, P, I, I, I, I, I, P, S, P]),
        "wam_pack_block_bytes": (S, [CFG]),
        "wam_pack_block": (I, [CFG, ctypes.POINTER(wam_block_weights), P, S, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(x):
    """Device/host pointer of a torch tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(st: int):
    if st != WAM_OK:
        raise WamError(st, load().wam_last_error().decode())


def _f32_host(vals):
    arr = (ctypes.c_float * len(vals))(*[float(v) for v in vals])
    return ctypes.cast(arr, ctypes.c_void_p).value, arr


def wam_workspace_bytes(cfg: wam_config, n_chunks: int) -> int:
    return int(load().wam_workspace_bytes(ctypes.byref(cfg), n_chunks))


def wam_ctx_set_state(cfg, w, state, ctx: wam_ctx_kv, ws, stream=None):
    _check(load().wam_ctx_set_state(ctypes.byref(cfg), ctypes.byref(w), _ptr(state), ctypes.byref(ctx), _ptr(ws),
                                    _nbytes(ws), _stream(stream)))


def wam_ctx_build(cfg, w, txt, img, ctx: wam_ctx_kv, ws, stream=None, state=None):
    _check(load().wam_ctx_build(ctypes.byref(cfg), ctypes.byref(w), _ptr(txt), _ptr(img), _ptr(state),
                                ctypes.byref(ctx), _ptr(ws), _nbytes(ws), _stream(stream)))


def wam_time_embed(cfg, w, t, e, e6, ws, stream=None):
    tp, keep = _f32_host(t)
    _check(load().wam_time_embed(ctypes.byref(cfg), ctypes.byref(w), tp, len(t), _ptr(e), _ptr(e6), _ptr(ws),
                                 _nbytes(ws), _stream(stream)))
    del keep


def wam_dit_stack_fwd(cfg, w, cache: wam_kv_cache, ctx: wam_ctx_kv, n_chunks, x_video, x_action, t_video, t_action,
                      start_frame, v_video, v_action, ws, stream=None):
    tvp, k1 = _f32_host(t_video)
    tap, k2 = _f32_host(t_action)
    _check(load().wam_dit_stack_fwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), ctypes.byref(ctx),
                                    n_chunks, _ptr(x_video), _ptr(x_action), tvp, tap, start_frame, _ptr(v_video),
                                    _ptr(v_action), _ptr(ws), _nbytes(ws), _stream(stream)))
    del k1, k2


def wam_kv_append(cfg, w, cache: wam_kv_cache, ctx: wam_ctx_kv, x_video, x_action, start_frame, ws, stream=None):
    _check(load().wam_kv_append(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(cache), ctypes.byref(ctx),
                                _ptr(x_video), _ptr(x_action), start_frame, _ptr(ws), _nbytes(ws), _stream(stream)))


def wam_dit_block_fwd(cfg, bw: wam_block_weights, layer, cache, ctx, h, e6, n_chunks, start_frame, ws, stream=None,
                      commit=False):
    _check(load().wam_dit_block_fwd(ctypes.byref(cfg), ctypes.byref(bw), layer, ctypes.byref(cache),
                                    ctypes.byref(ctx), _ptr(h), _ptr(e6), n_chunks, start_frame, 1 if commit else 0,
                                    _ptr(ws), _nbytes(ws), _stream(stream)))


def wam_flow_step(x_video, x_action, v_video, v_action, branches, guidance, n_video, n_action, dt_video, dt_action,
                  g_video=None, g_action=None, prev_video=None, cos_parts=None, ws=None, stream=None):
    _check(load().wam_flow_step(_ptr(x_video), _ptr(x_action), _ptr(v_video), _ptr(v_action), branches,
                                float(guidance), n_video, n_action, float(dt_video), float(dt_action), _ptr(g_video),
                                _ptr(g_action), _ptr(prev_video), _ptr(cos_parts), _ptr(ws), _nbytes(ws),
                                _stream(stream)))


def wam_flow_step_noalloc(x_video, x_action, v_video, v_action, branches, guidance, n_video, n_action, dt_video,
                          dt_action, g_video=None, g_action=None, prev_video=None, cos_parts=None, stream=None):
    _check(load().wam_flow_step_noalloc(_ptr(x_video), _ptr(x_action), _ptr(v_video), _ptr(v_action), branches,
                                        float(guidance), n_video, n_action, float(dt_video), float(dt_action),
                                        _ptr(g_video), _ptr(g_action), _ptr(prev_video), _ptr(cos_parts),
                                        _stream(stream)))


def wam_denoise_chunk(cfg, weights, cache, ctx, x_video, x_action, grid, guidance, tau, v_video, v_action, g_video,
                      g_action, cos_parts, ws, start_frame=0, max_consecutive_reuse=-1, stream=None):
    """Returns (number of DiT passes, list of per-step reuse flags). ``grid`` is a host sequence of
    n_steps + 1 times."""
    n = len(grid) - 1
    g = (ctypes.c_float * (n + 1))(*[float(t) for t in grid])
    calls = ctypes.c_int(0)
    flags = (ctypes.c_ubyte * max(n, 1))()
    _check(load().wam_denoise_chunk(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(ctx),
                                    _ptr(x_video), _ptr(x_action), ctypes.cast(g, ctypes.c_void_p), n, float(guidance),
                                    float(tau), int(max_consecutive_reuse), int(start_frame), _ptr(v_video),
                                    _ptr(v_action), _ptr(g_video), _ptr(g_action), _ptr(cos_parts), _ptr(ws),
                                    _nbytes(ws), _stream(stream), ctypes.cast(ctypes.byref(calls), ctypes.c_void_p),
                                    ctypes.cast(flags, ctypes.c_void_p)))
    return calls.value, [bool(flags[i]) for i in range(n)]


def wam_denoise_chunk_replay(cfg, weights, cache, ctx, x_video, x_action, grid, guidance, replay, v_video, v_action,
                             g_video, g_action, cos_parts, ws, start_frame=0, want_cosines=True, stream=None):
    """Euler loop following the host reuse mask ``replay`` (n_steps flags). Returns (number of DiT passes,
    per-step cosines the decision rule would compare, NaN where none; None without want_cosines)."""
    n = len(grid) - 1
    g = (ctypes.c_float * (n + 1))(*[float(t) for t in grid])
    mask = (ctypes.c_ubyte * max(n, 1))(*[1 if f else 0 for f in replay])
    calls = ctypes.c_int(0)
    cos = (ctypes.c_float * max(n, 1))()
    _check(load().wam_denoise_chunk_replay(
        ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(ctx), _ptr(x_video),
        _ptr(x_action), ctypes.cast(g, ctypes.c_void_p), n, float(guidance), ctypes.cast(mask, ctypes.c_void_p),
        int(start_frame), _ptr(v_video), _ptr(v_action), _ptr(g_video), _ptr(g_action), _ptr(cos_parts), _ptr(ws),
        _nbytes(ws), _stream(stream), ctypes.cast(ctypes.byref(calls), ctypes.c_void_p),
        ctypes.cast(cos, ctypes.c_void_p) if want_cosines else None))
    return calls.value, ([float(cos[i]) for i in range(n)] if want_cosines else None)


def wam_denoise_chunk_unipc(cfg, weights, cache, ctx, x_video, x_action, grid, guidance, tau, v_video, v_action,
                            g_video, g_action, cos_parts, state, ws, order=2, corrector=True, start_frame=0,
                            max_consecutive_reuse=-1, stream=None):
    """UniPC variant of ``wam_denoise_chunk``; ``state`` holds 5 x (video + action) floats."""
    n = len(grid) - 1
    g = (ctypes.c_float * (n + 1))(*[float(t) for t in grid])
    calls = ctypes.c_int(0)
    flags = (ctypes.c_ubyte * max(n, 1))()
    _check(load().wam_denoise_chunk_unipc(
        ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(cache), ctypes.byref(ctx), _ptr(x_video),
        _ptr(x_action), ctypes.cast(g, ctypes.c_void_p), n, float(guidance), float(tau), int(max_consecutive_reuse),
        int(start_frame), int(order), 1 if corrector else 0, _ptr(v_video), _ptr(v_action), _ptr(g_video),
        _ptr(g_action), _ptr(cos_parts), _ptr(state), _ptr(ws), _nbytes(ws), _stream(stream),
        ctypes.cast(ctypes.byref(calls), ctypes.c_void_p), ctypes.cast(flags, ctypes.c_void_p)))
    return calls.value, [bool(flags[i]) for i in range(n)]


def wam_op_linear(dtype, A, lda, W, ldw, bias, C, ldc, M, N, K, act=0, ws=None, stream=None):
    """``ws``: optional device scratch tensor for split-K partial products (None: no split)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().wam_op_linear(dtype, _ptr(A), lda, _ptr(W), ldw, _ptr(bias), _ptr(C), ldc, M, N, K, act,
                                _ptr(ws), nbytes, _stream(stream)))


def wam_op_split_finish(part, splits, M, N, bias, h, e6, mod_gate, gate_idx, mod_norm, shift_idx, scale_idx, y,
                        rms=False, eps=1e-6, stream=None):
    _check(load().wam_op_split_finish(_ptr(part), splits, M, N, _ptr(bias), _ptr(h), _ptr(e6), _ptr(mod_gate),
                                      gate_idx, _ptr(mod_norm), shift_idx, scale_idx, 1 if rms else 0, float(eps),
                                      _ptr(y), _stream(stream)))


def wam_op_modulated_norm(x, M, D, e6, mod, shift_idx, scale_idx, y, rms=False, eps=1e-6, stream=None):
    _check(load().wam_op_modulated_norm(_ptr(x), M, D, _ptr(e6), _ptr(mod), shift_idx, scale_idx, 1 if rms else 0,
                                        float(eps), _ptr(y), _stream(stream)))


def wam_op_qkv_cache(qkv, br, rows, Lq, Lv, H, d, g_q, g_k, eps, rope, q_out, k_cache, v_cache, cap, row0=0,
                     stream=None):
    _check(load().wam_op_qkv_cache(_ptr(qkv), br, rows, Lq, Lv, H, d, _ptr(g_q), _ptr(g_k), float(eps), _ptr(rope),
                                   _ptr(q_out), _ptr(k_cache), _ptr(v_cache), cap, row0, _stream(stream)))


def wam_mx_quantize(dtype, src, ld, rows, cols, codes, ldq, scales, stream=None):
    _check(load().wam_mx_quantize(dtype, _ptr(src), ld, rows, cols, _ptr(codes), ldq, _ptr(scales), _stream(stream)))


def wam_weights_for_embodiment(w: wam_weights, id: int) -> wam_weights:
    out = wam_weights()
    _check(load().wam_weights_for_embodiment(ctypes.byref(w), id, ctypes.byref(out)))
    return out


def wam_mx_block_bytes(cfg: wam_config) -> int:
    return int(load().wam_mx_block_bytes(ctypes.byref(cfg)))


def wam_mx_pack_block(cfg: wam_config, bw: wam_block_weights, dst, stream=None):
    nbytes = dst.numel() * dst.element_size()
    _check(load().wam_mx_pack_block(ctypes.byref(cfg), ctypes.byref(bw), _ptr(dst), nbytes, _stream(stream)))


def wam_mx4_quantize(dtype, src, ld, rows, cols, codes, ldq, scales, stream=None):
    _check(load().wam_mx4_quantize(dtype, _ptr(src), ld, rows, cols, _ptr(codes), ldq, _ptr(scales), _stream(stream)))


def wam_pack_weight(W, ldw, N, K, dst, stream=None):
    """Fragment-packed copy of the bf16 matrix W [N][ldw] into dst (N * K bf16)."""
    _check(load().wam_pack_weight(_ptr(W), ldw, N, K, _ptr(dst), _stream(stream)))


def wam_op_linear_packed(A, lda, Wp, bias, C, ldc, M, N, K, act=0, ws=None, stream=None):
    """bf16 product with a fragment-packed weight (from wam_pack_weight)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().wam_op_linear_packed(_ptr(A), lda, _ptr(Wp), _ptr(bias), _ptr(C), ldc, M, N, K, act, _ptr(ws), nbytes,
                                       _stream(stream)))


def wam_pack_block_bytes(cfg: wam_config) -> int:
    return int(load().wam_pack_block_bytes(ctypes.byref(cfg)))


def wam_pack_block(cfg: wam_config, bw: wam_block_weights, dst, stream=None):
    nbytes = dst.numel() * dst.element_size()
    _check(load().wam_pack_block(ctypes.byref(cfg), ctypes.byref(bw), _ptr(dst), nbytes, _stream(stream)))


def wam_op_linear_mx(A, A_scales, lda, W, W_scales, ldw, bias, C, ldc, M, N, K, act=0, ws=None, stream=None,
                     w_format=WAM_MX_E4M3):
    """MXFP8 product: uint8 code / scale tensors in, bf16 C out."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().wam_op_linear_mx(_ptr(A), _ptr(A_scales), lda, _ptr(W), _ptr(W_scales), ldw, w_format, _ptr(bias),
                                   _ptr(C), ldc,
                                   M, N, K, act, _ptr(ws), nbytes, _stream(stream)))


def wam_op_attention(dtype, Q, K, Vt, O, br, heads, head_dim, Lq, k_rows, v_stride, kv_base, chunk_q, kv_total,
                     ws=None, stream=None):
    """``ws``: optional device scratch tensor for key-split partial outputs (None: no split)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().wam_op_attention(dtype, _ptr(Q), _ptr(K), _ptr(Vt), _ptr(O), br, heads, head_dim, Lq, k_rows,
                                   v_stride, kv_base, chunk_q, kv_total, _ptr(ws), nbytes, _stream(stream)))


def wam_kv_evict(cfg, cache: wam_kv_cache, drop_rows: int, frame_shift: int, stream=None):
    _check(load().wam_kv_evict(ctypes.byref(cfg), ctypes.byref(cache), drop_rows, frame_shift, _stream(stream)))


def wam_kv_reset(cache: wam_kv_cache):
    load().wam_kv_reset(ctypes.byref(cache))


def wam_last_error() -> str:
    return load().wam_last_error().decode()


def wam_op_attention_mx(Q, Qs, K, Ks, Vt, Vs, O, br, heads, Lq, k_rows, v_stride, kv_base, chunk_q, kv_total,
                        stream=None):
    _check(load().wam_op_attention_mx(_ptr(Q), _ptr(Qs), _ptr(K), _ptr(Ks), _ptr(Vt), _ptr(Vs), _ptr(O), br, heads,
                                      Lq, k_rows, v_stride, kv_base, chunk_q, kv_total, _stream(stream)))


def wam_qkv_timer_config(layer: int, max_samples: int = 1):
    """Record HIP events around block ``layer``'s QKV product in later passes (layer < 0: off)."""
    _check(load().wam_qkv_timer_config(layer, max_samples))


def wam_mfma_peak_probe(out, workgroups: int, iters: int, stream=None):
    """Back-to-back bf16 MFMAs on every SIMD (see include/wam.h); ``out`` holds workgroups x 256 floats."""
    _check(load().wam_mfma_peak_probe(_ptr(out), workgroups, iters, _stream(stream)))


def wam_qkv_timer_read(cap: int = 4096):
    """Durations in ms of the samples recorded since the last read (waits for their events)."""
    buf = (ctypes.c_float * max(cap, 1))()
    n = ctypes.c_int(0)
    _check(load().wam_qkv_timer_read(buf, cap, ctypes.byref(n)))
    return [float(buf[i]) for i in range(min(n.value, cap))]


def _nbytes(ws):
    if ws is None:
        return 0
    if isinstance(ws, int):
        raise TypeError("pass the workspace as a tensor so its size is known")
    return ws.numel() * ws.element_size()
