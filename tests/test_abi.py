"""The C-ABI library: it loads, exports every function ``include/wam.h`` declares, and rejects bad
arguments on the host before anything is enqueued (no GPU needed: validation makes no HIP call)."""
import ctypes
import os
import re

import pytest

import world_action_video_amd as wam
from synth.workloads import WORKLOADS
from world_action_video_amd.build import OUT

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(OUT):
        from world_action_video_amd.build import build
        build()
    return wam.load()


def _declared():
    text = open(os.path.join(ROOT, "include", "wam.h")).read()
    return sorted(set(re.findall(r"^\s*(?:wam_status|size_t|void|const char \*)\s*\*?\s*(wam_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree():
    assert _declared() == sorted(wam.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name


def _cfg(wid=1, dtype="bf16"):
    from world_action_video_amd.device import make_config
    return make_config(WORKLOADS[wid], dtype)


def test_workspace_bytes_host_only():
    _lib()
    c1 = _cfg(1)
    b1 = wam.wam_workspace_bytes(c1, 1)
    b2 = wam.wam_workspace_bytes(c1, 2)
    assert 0 < b1 < b2
    assert wam.wam_workspace_bytes(c1, 0) == 0 and wam.wam_workspace_bytes(c1, 9) == 0
    c3 = _cfg(3)
    M = 2 * 464
    assert wam.wam_workspace_bytes(c3, 1) >= M * 5120 * 4 + M * 13824 * 2
    bad = _cfg(1)
    bad.head_dim = 96
    assert wam.wam_workspace_bytes(bad, 1) == 0


def test_validation_rejects_before_launch():
    lib = _lib()
    c = _cfg(1)
    st = lib.wam_dit_stack_fwd(None, None, None, None, 1, None, None, None, None, 0, None, None, None, 0, None)
    assert st == wam.WAM_E_ARG and "config" in wam.wam_last_error()
    st = lib.wam_dit_stack_fwd(ctypes.byref(c), None, None, None, 1, None, None, None, None, 0, None, None, None, 0, None)
    assert st == wam.WAM_E_ARG and "weights" in wam.wam_last_error()
    bad = _cfg(1)
    bad.dim = 250
    st = lib.wam_dit_stack_fwd(ctypes.byref(bad), None, None, None, 1, None, None, None, None, 0, None, None, None, 0,
                               None)
    assert st == wam.WAM_E_SHAPE
    # capacity overflow is reported as such, with nothing launched (all pointers are fake host values)
    w = wam.wam_weights()
    blocks = (wam.wam_block_weights * c.layers)()
    for b in blocks:
        for f in wam.BLOCK_FIELDS:
            setattr(b, f, 0x1000)
    w.blocks = ctypes.cast(blocks, ctypes.POINTER(wam.wam_block_weights))
    for f in wam.GLOBAL_FIELDS:
        setattr(w, f, 0x1000)
    kv = wam.wam_kv_cache(0x1000, 0x1000, 2, 128, 0)
    cx = wam.wam_ctx_kv(0x1000, 0x1000, 2, 32, 64)
    st = lib.wam_dit_stack_fwd(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(cx), 1, 0x1000, 0x1000,
                               None, None, 0, 0x1000, 0x1000, 0x1000, 1 << 30, None)
    assert st == wam.WAM_E_CAPACITY
    kv = wam.wam_kv_cache(0x1000, 0x1000, 2, 100, 0)
    st = lib.wam_kv_append(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(cx), 0x1000, 0x1000, 0,
                           0x1000, 1 << 30, None)
    assert st == wam.WAM_E_SHAPE and kv.length == 0
    cx_bad = wam.wam_ctx_kv(0x1000, 0x1000, 2, 31, 64)
    kv = wam.wam_kv_cache(0x1000, 0x1000, 2, 512, 0)
    st = lib.wam_kv_append(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(cx_bad), 0x1000, 0x1000, 0,
                           0x1000, 1 << 30, None)
    assert st == wam.WAM_E_SHAPE and kv.length == 0
    st = lib.wam_kv_append(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(cx), 0x1000, 0x1000, 0,
                           0x1000, 16, None)
    assert st == wam.WAM_E_ARG and "workspace" in wam.wam_last_error() and kv.length == 0
    blocks[c.layers - 1].g_q = 0x1008   # the kernels read vectors with 16-byte loads
    st = lib.wam_kv_append(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(cx), 0x1000, 0x1000, 0,
                           0x1000, 1 << 30, None)
    assert st == wam.WAM_E_ARG and "g_q is not 16-byte aligned" in wam.wam_last_error() and kv.length == 0
    blocks[c.layers - 1].g_q = 0x1000
    blocks[c.layers - 1].w_ff2 = None
    st = lib.wam_kv_append(ctypes.byref(c), ctypes.byref(w), ctypes.byref(kv), ctypes.byref(cx), 0x1000, 0x1000, 0,
                           0x1000, 1 << 30, None)
    assert st == wam.WAM_E_ARG and "w_ff2" in wam.wam_last_error() and kv.length == 0


def test_op_validation():
    lib = _lib()
    assert lib.wam_op_linear(0, 0x1000, 64, 0x1000, 64, None, 0x1000, 64, 4, 4, 60, 0, None, 0, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_linear(0, None, 64, 0x1000, 64, None, 0x1000, 64, 4, 4, 64, 0, None, 0, None) == wam.WAM_E_ARG
    assert lib.wam_op_attention(0, 0x1000, 0x1000, 0x1000, 0x1000, 1, 1, 96, 8, 8, 8, 0, 0, 8, None, 0,
                                None) == wam.WAM_E_SHAPE
    assert lib.wam_op_attention(0, 0x1000, 0x1000, 0x1000, 0x1000, 1, 1, 64, 8, 8, 12, 0, 0, 12, None, 0,
                                None) == wam.WAM_E_SHAPE
    assert lib.wam_op_attention(0, 0x1000, 0x1000, 0x1000, 0x1000, 1, 1, 64, 8, 8, 8, 0, 0, 8, 0x1010, 4096,
                                None) == wam.WAM_E_ARG
    assert lib.wam_flow_step(0x1000, 0x1000, 0x1000, 0x1000, 3, 5.0, 4, 4, 0.1, 0.1, None, None, None, None, None, 0,
                             None) == wam.WAM_E_SHAPE
    assert lib.wam_flow_step(0x1000, 0x1000, 0x1000, 0x1000, 2, 5.0, 4, 4, 0.1, 0.1, None, None, 0x1000, None, None, 0,
                             None) == wam.WAM_E_ARG
    # the allocation-free variant validates the same way before touching its scratch
    assert lib.wam_flow_step_noalloc(0x1000, 0x1000, 0x1000, 0x1000, 3, 5.0, 4, 4, 0.1, 0.1, None, None, None, None,
                                     None) == wam.WAM_E_SHAPE
    assert lib.wam_flow_step_noalloc(0x1000, 0x1000, 0x1000, 0x1000, 2, 5.0, 4, 4, 0.1, 0.1, None, None, 0x1000, None,
                                     None) == wam.WAM_E_ARG
    assert lib.wam_flow_step_noalloc(None, 0x1000, 0x1000, 0x1000, 2, 5.0, 4, 4, 0.1, 0.1, None, None, None, None,
                                     None) == wam.WAM_E_ARG


def test_attention_mx_validation():
    """The MXFP8 attention op rejects bad sizes and alignment on the host (fake pointers, nothing
    launched)."""
    lib = _lib()
    ok = (0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    assert lib.wam_op_attention_mx(*ok, 2, 4, 100, 300, 300, 0, 0, 300, None) == wam.WAM_E_SHAPE   # v_stride % 64
    assert lib.wam_op_attention_mx(*ok, 2, 4, 100, 300, 256, 0, 0, 300, None) == wam.WAM_E_SHAPE   # v_stride < 320
    assert lib.wam_op_attention_mx(*ok, 2, 4, 100, 200, 320, 0, 0, 300, None) == wam.WAM_E_SHAPE   # k_rows < kv_total
    assert lib.wam_op_attention_mx(*ok, 2, 4, 0, 300, 320, 0, 0, 300, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_attention_mx(*ok, 2, 4, 100, 300, 320, 0, -1, 300, None) == wam.WAM_E_SHAPE
    bad = (0x1008,) + ok[1:]
    assert lib.wam_op_attention_mx(*bad, 2, 4, 100, 300, 320, 0, 0, 300, None) == wam.WAM_E_ARG
    assert lib.wam_op_attention_mx(None, *ok[1:], 2, 4, 100, 300, 320, 0, 0, 300, None) == wam.WAM_E_ARG
    assert "aligned" in wam.wam_last_error() or "NULL" in wam.wam_last_error()


def test_qkv_timer_host_side():
    """The measurement hook's host-side paths: disabling, bad sample counts and reads with nothing
    recorded make no HIP call (enabling creates events, which needs a GPU)."""
    lib = _lib()
    assert lib.wam_qkv_timer_config(-1, 0) == wam.WAM_OK
    assert lib.wam_qkv_timer_config(3, 0) == wam.WAM_E_ARG and "max_samples" in wam.wam_last_error()
    assert lib.wam_qkv_timer_config(3, 5000) == wam.WAM_E_ARG
    n = ctypes.c_int(-1)
    assert lib.wam_qkv_timer_read(None, 0, ctypes.byref(n)) == wam.WAM_OK and n.value == 0
    assert lib.wam_qkv_timer_read(None, 4, ctypes.byref(n)) == wam.WAM_E_ARG
    assert lib.wam_qkv_timer_read(None, 0, None) == wam.WAM_E_ARG
    assert wam.wam_qkv_timer_read(8) == []


def test_mx_validation():
    """MXFP8 entry points reject bad shapes and alignment on the host (fake pointers, nothing launched)."""
    lib = _lib()
    P = 0x1000
    # quantiser: cols not a multiple of 32, ldq not a multiple of 16, src misaligned, unknown dtype
    assert lib.wam_mx_quantize(0, P, 48, 4, 48, P, 48, P, None) == wam.WAM_E_SHAPE
    assert lib.wam_mx_quantize(0, P, 64, 4, 64, P, 72, P, None) == wam.WAM_E_SHAPE
    assert lib.wam_mx_quantize(1, P + 4, 64, 4, 64, P, 64, P, None) == wam.WAM_E_ARG
    assert lib.wam_mx_quantize(7, P, 64, 4, 64, P, 64, P, None) == wam.WAM_E_ARG
    # product: K not a multiple of 128, N not a multiple of 4, odd SwiGLU pitch, scale misaligned, NULL operand
    args = lambda **kw: [kw.get(n, d) for n, d in (  # noqa: E731
        ("A", P), ("As", P), ("lda", 256), ("W", P), ("Ws", P), ("ldw", 256), ("wf", 0), ("bias", None), ("C", P),
        ("ldc", 64),
        ("M", 8), ("N", 64), ("K", 256), ("act", 0), ("ws", None), ("wsb", 0), ("s", None))]
    assert lib.wam_op_linear_mx(*args(K=192, lda=192, ldw=192)) == wam.WAM_E_SHAPE
    assert lib.wam_op_linear_mx(*args(N=62)) == wam.WAM_E_SHAPE
    assert lib.wam_op_linear_mx(*args(N=60, act=2, ldc=30)) == wam.WAM_E_SHAPE
    assert lib.wam_op_linear_mx(*args(Ws=P + 2)) == wam.WAM_E_ARG
    assert lib.wam_op_linear_mx(*args(As=None)) == wam.WAM_E_ARG
    assert lib.wam_op_linear_mx(*args(act=3)) == wam.WAM_E_ARG
    assert lib.wam_op_linear_mx(*args(wf=2)) == wam.WAM_E_ARG
    assert lib.wam_op_linear_mx(*args(wf=1, ldw=112)) == wam.WAM_E_SHAPE     # e2m1 rows need K / 2 = 128 bytes
    assert lib.wam_mx4_quantize(0, P, 64, 4, 64, P, 16, P, None) == wam.WAM_E_SHAPE   # ldq < cols / 2


def test_image_cross_attention_validation():
    """The separate image cross-attention variant needs image tokens, the image projections and a
    condition value stride that holds the image key tiles (checked before anything runs)."""
    lib = _lib()
    from world_action_video_amd.device import make_config
    w = WORKLOADS[1].with_(ctx_img_len=0, variant=8)
    c = make_config(w, "f32")
    assert lib.wam_workspace_bytes(ctypes.byref(c), 1) == 0
    assert "image" in wam.wam_last_error()
    c = make_config(WORKLOADS[1].with_(ctx_img_len=16, variant=8), "f32")
    assert lib.wam_workspace_bytes(ctypes.byref(c), 1) > 0


def test_state_rows_validation():
    """State rows: state_dim a multiple of 64, no combination with the separate image attention,
    and wam_ctx_set_state refused without state rows (checked before anything runs)."""
    lib = _lib()
    from world_action_video_amd.device import make_config
    c = make_config(WORKLOADS[1].with_(ctx_state_len=1), "f32")
    assert lib.wam_workspace_bytes(ctypes.byref(c), 1) > 0
    c = make_config(WORKLOADS[1].with_(ctx_state_len=1, state_dim=40), "f32")
    assert lib.wam_workspace_bytes(ctypes.byref(c), 1) == 0 and "state_dim" in wam.wam_last_error()
    c = make_config(WORKLOADS[1].with_(ctx_state_len=1, ctx_img_len=16, variant=8), "f32")
    assert lib.wam_workspace_bytes(ctypes.byref(c), 1) == 0 and "state rows" in wam.wam_last_error()
    c = make_config(WORKLOADS[1], "f32")
    w = wam.wam_weights()
    cx = wam.wam_ctx_kv(0x1000, 0x1000, 2, 32, 64)
    assert lib.wam_ctx_set_state(ctypes.byref(c), ctypes.byref(w), 0x1000, ctypes.byref(cx), 0x1000, 1 << 30,
                                 None) == wam.WAM_E_SHAPE


def test_embodiment_routing_is_host_only():
    """wam_weights_for_embodiment swaps the action encoder / decoder pointers and nothing else."""
    _lib()
    w = wam.wam_weights()
    for i, name in enumerate(wam.GLOBAL_FIELDS):
        setattr(w, name, 0x1000 + 0x100 * i)
    table = (wam.wam_action_io * 2)()
    for e in range(2):
        for j, name in enumerate(("ae_w", "ae_b", "ao_w", "ao_b")):
            setattr(table[e], name, 0x900000 + 0x1000 * e + 0x10 * j)
    w.embodiments = ctypes.cast(table, ctypes.POINTER(wam.wam_action_io))
    w.n_embodiments = 2
    r = wam.wam_weights_for_embodiment(w, 1)
    for name in wam.GLOBAL_FIELDS:
        want = getattr(table[1], name) if name in ("ae_w", "ae_b", "ao_w", "ao_b") else getattr(w, name)
        assert getattr(r, name) == want, name
    assert r.n_embodiments == 2
    with pytest.raises(wam.WamError, match="embodiment 2"):
        wam.wam_weights_for_embodiment(w, 2)
    with pytest.raises(wam.WamError):
        wam.wam_weights_for_embodiment(w, -1)
    w.n_embodiments = 0
    with pytest.raises(wam.WamError):
        wam.wam_weights_for_embodiment(w, 0)


def test_empty_and_oversized_products():
    """M = 0 launches nothing and succeeds; operands past the 32-bit buffer offsets are rejected as a
    shape error before anything runs (fake pointers, no GPU needed)."""
    lib = _lib()
    P = 0x1000
    assert lib.wam_op_linear(0, P, 64, P, 64, None, P, 64, 0, 64, 64, 0, None, 0, None) == wam.WAM_OK
    assert lib.wam_op_linear(0, P, 8192, P, 8192, None, P, 64, 300000, 64, 8192, 0, None, 0, None) == wam.WAM_E_SHAPE
    assert "2 GiB" in wam.wam_last_error()
    assert lib.wam_op_linear(1, P, 8192, P, 8192, None, P, 300000, 64, 300000, 8192, 0, None, 0, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_linear_mx(P, P, 256, P, P, 256, 0, None, P, 64, 0, 64, 256, 0, None, 0, None) == wam.WAM_OK
    assert lib.wam_op_linear_mx(P, P, 16384, P, P, 16384, 0, None, P, 64, 140000, 64, 16384, 0, None, 0,
                                None) == wam.WAM_E_SHAPE
    assert lib.wam_op_attention(0, P, P, P, P, 1, 1, 64, 0, 64, 64, 0, 0, 8, None, 0, None) == wam.WAM_OK


def test_kv_reset_is_host_only():
    _lib()
    kv = wam.wam_kv_cache(0x1000, 0x1000, 2, 512, 464)
    wam.wam_kv_reset(kv)
    assert kv.length == 0


def test_denoise_chunk_validation():
    """The denoising loop checks its own arguments, and its first DiT pass checks the rest, before
    anything is enqueued."""
    lib = _lib()
    c = _cfg(1)
    F = ctypes.c_float
    grid = (F * 3)(0.0, 0.5, 1.0)
    P = 0x1000
    args = lambda g, n, gv=P, cosp=P: (ctypes.byref(c), None, None, None, P, P, g, n, F(5.0), F(2.0), -1, 0, P, P,  # noqa
                                       gv, P, cosp, P, 1 << 30, None, None, None)
    assert lib.wam_denoise_chunk(*args(None, 2)) == wam.WAM_E_ARG and "grid" in wam.wam_last_error()
    assert lib.wam_denoise_chunk(*args(grid, 0)) == wam.WAM_E_ARG
    nan_grid = (F * 3)(0.0, float("nan"), 1.0)
    assert lib.wam_denoise_chunk(*args(nan_grid, 2)) == wam.WAM_E_ARG and "non-finite" in wam.wam_last_error()
    assert lib.wam_denoise_chunk(*args(grid, 2, gv=None)) == wam.WAM_E_ARG
    # valid loop arguments: the first DiT pass rejects the missing weights
    assert lib.wam_denoise_chunk(*args(grid, 2)) == wam.WAM_E_ARG and "weights" in wam.wam_last_error()


def test_kv_evict_validation():
    """Eviction keeps whole chunks and rejects bad requests on the host; nothing changes then."""
    lib = _lib()
    c = _cfg(1)
    lq = WORKLOADS[1].chunk_tokens
    kv = wam.wam_kv_cache(0x1000, 0x1000, 2, 512, 2 * lq)
    assert lib.wam_kv_evict(ctypes.byref(c), ctypes.byref(kv), lq - 8, 2, None) == wam.WAM_E_SHAPE
    assert kv.length == 2 * lq
    assert lib.wam_kv_evict(ctypes.byref(c), ctypes.byref(kv), 3 * lq, 2, None) == wam.WAM_E_SHAPE
    assert lib.wam_kv_evict(ctypes.byref(c), None, lq, 2, None) == wam.WAM_E_ARG
    bad = wam.wam_kv_cache(0x1008, 0x1000, 2, 512, 2 * lq)
    assert lib.wam_kv_evict(ctypes.byref(c), ctypes.byref(bad), lq, 2, None) == wam.WAM_E_ARG
    assert lib.wam_kv_evict(ctypes.byref(c), ctypes.byref(kv), 0, 2, None) == wam.WAM_OK and kv.length == 2 * lq


def test_denoise_chunk_unipc_validation():
    """The UniPC loop checks its order, state and grid before anything is enqueued."""
    lib = _lib()
    c = _cfg(1)
    F = ctypes.c_float
    P = 0x1000
    grid = (F * 3)(0.0, 0.5, 1.0)

    def call(g, order, state=P):
        return lib.wam_denoise_chunk_unipc(ctypes.byref(c), None, None, None, P, P, g, 2, F(5.0), F(2.0), -1, 0, order,
                                           1, P, P, P, P, P, state, P, 1 << 30, None, None, None)
    assert call(grid, 0) == wam.WAM_E_ARG and "order" in wam.wam_last_error()
    assert call(grid, 4) == wam.WAM_E_ARG and "order" in wam.wam_last_error()
    assert call(grid, 2, state=None) == wam.WAM_E_ARG and "state" in wam.wam_last_error()
    flat = (F * 3)(0.0, 0.5, 0.5)
    assert call(flat, 2) == wam.WAM_E_ARG and "increase" in wam.wam_last_error()
    outside = (F * 3)(0.0, 0.5, 1.5)
    assert call(outside, 2) == wam.WAM_E_ARG
    # valid loop arguments: the first DiT pass rejects the missing weights
    assert call(grid, 2) == wam.WAM_E_ARG and "weights" in wam.wam_last_error()


def test_denoise_chunk_replay_validation():
    """The replay loop rejects a NULL mask and a mask that skips step 0 or 1, before any launch."""
    import ctypes
    lib = _lib()
    c = _cfg(1)
    wts = wam.wam_weights()
    kv = wam.wam_kv_cache(0x1000, 0x1000, 2, 256, 0)
    cx = wam.wam_ctx_kv(0x1000, 0x1000, 2, 32, 64)
    grid = (ctypes.c_float * 3)(0.0, 0.5, 1.0)
    for mask in (None, (ctypes.c_ubyte * 2)(1, 0), (ctypes.c_ubyte * 2)(0, 1)):
        st = lib.wam_denoise_chunk_replay(ctypes.byref(c), ctypes.byref(wts), ctypes.byref(kv), ctypes.byref(cx),
                                          0x1000, 0x1000, ctypes.cast(grid, ctypes.c_void_p), 2, 5.0,
                                          None if mask is None else ctypes.cast(mask, ctypes.c_void_p), 0, 0x1000,
                                          0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 1 << 30, None, None, None)
        assert st == wam.WAM_E_ARG, st



def test_row_op_validation():
    """The kernel-level row ops reject bad arguments before any launch, and an empty call succeeds
    (fake pointers: nothing is dereferenced, no GPU needed)."""
    lib = _lib()
    P = 0x1000
    # split finish: part, splits, M, N, bias, h, e6, mod_gate, gate_idx, mod_norm, shift, scale, rms, eps, y
    ok = (P, 3, 0, 5120, None, P, P, P, 5, P, 0, 1, 0, 1e-6, P, None)
    assert lib.wam_op_split_finish(*ok) == wam.WAM_OK
    assert lib.wam_op_split_finish(P, 1, 8, 5120, None, P, P, P, 5, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_split_finish(P, 5, 8, 5120, None, P, P, P, 5, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_split_finish(P, 3, 8, 5122, None, P, P, P, 5, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_split_finish(P, 3, 8, 8196, None, P, P, P, 5, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_split_finish(P, 3, 8, 5120, None, P, P, None, 5, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_ARG
    assert lib.wam_op_split_finish(P, 3, 8, 5120, None, P, P, P, 6, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_ARG
    assert lib.wam_op_split_finish(P, 3, 8, 5120, None, P, P, P, 5, P, 0, 1, 0, 0.0, P, None) == wam.WAM_E_ARG
    assert lib.wam_op_split_finish(P + 4, 3, 8, 5120, None, P, P, P, 5, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_ARG
    # without a gate the gate offsets may be NULL
    assert lib.wam_op_split_finish(P, 3, 0, 5120, None, P, P, None, -1, P, 3, 4, 0, 1e-6, P, None) == wam.WAM_OK
    # modulated norm: x, M, D, e6, mod, shift, scale, rms, eps, y
    assert lib.wam_op_modulated_norm(P, 0, 5120, P, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_OK
    assert lib.wam_op_modulated_norm(P, 8, 5118, P, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_modulated_norm(P, 8, 5120, P, P, -1, 1, 0, 1e-6, P, None) == wam.WAM_E_ARG
    assert lib.wam_op_modulated_norm(P, 8, 5120, None, P, 0, 1, 0, 1e-6, P, None) == wam.WAM_E_ARG
    # q/k/v: qkv, br, rows, Lq, Lv, H, d, g_q, g_k, eps, rope, q_out, k_cache, v_cache, cap, row0
    assert lib.wam_op_qkv_cache(P, 2, 0, 464, 440, 40, 128, P, P, 1e-6, P, P, P, P, 928, 0, None) == wam.WAM_OK
    assert lib.wam_op_qkv_cache(P, 2, 464, 464, 440, 40, 96, P, P, 1e-6, P, P, P, P, 928, 0, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_qkv_cache(P, 2, 464, 464, 440, 40, 128, P, P, 1e-6, P, P, P, P, 928, 472, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_qkv_cache(P, 2, 460, 464, 440, 40, 128, P, P, 1e-6, P, P, P, P, 928, 0, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_qkv_cache(P, 2, 464, 464, 470, 40, 128, P, P, 1e-6, P, P, P, P, 928, 0, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_qkv_cache(P, 2, 464, 464, 440, 80, 128, P, P, 1e-6, P, P, P, P, 928, 0, None) == wam.WAM_E_SHAPE
    assert lib.wam_op_qkv_cache(P, 2, 464, 464, 440, 40, 128, P, None, 1e-6, P, P, P, P, 928, 0, None) == wam.WAM_E_ARG
