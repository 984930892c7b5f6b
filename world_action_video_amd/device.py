"""Device-side buffers for the C ABI: weights, caches and workspace as torch tensors on one GPU.

torch is used here only to allocate device memory and to move the seeded inputs onto it; the
library computes everything. Weight values come from the ``synth`` package (the same values the
CPU oracle reads), so both sides see identical bf16-representable numbers.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

import synth
from synth.workloads import Workload, draw, global_tensors, is_matrix, layer_tensors

from . import (GLOBAL_FIELDS, WAM_BF16, WAM_F32, wam_action_io, wam_block_weights, wam_config,
               wam_ctx_kv, wam_kv_cache, wam_mx_block_bytes, wam_mx_pack_block, wam_pack_block, wam_pack_block_bytes,
               wam_weights, wam_weights_for_embodiment, wam_workspace_bytes)


def make_config(w: Workload, dtype: str = "bf16", branches: int | None = None) -> wam_config:
    c = wam_config()
    for f in ("dim", "heads", "head_dim", "ffn_dim", "layers", "freq_dim", "patch_dim", "action_dim",
              "action_tokens", "frames_per_chunk", "grid_h", "grid_w", "ctx_in_dim", "ctx_text_len", "ctx_img_len"):
        setattr(c, f, int(getattr(w, f)))
    c.branches = int(branches if branches is not None else w.branches)
    c.rope_theta = float(w.rope_theta)
    c.eps = float(w.eps)
    c.dtype = WAM_BF16 if dtype == "bf16" else WAM_F32
    c.variant = int(w.variant)
    c.precision = int(w.precision)
    c.ctx_state_len = int(w.ctx_state_len)
    c.state_dim = int(w.state_dim)
    return c


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_device(arr_f32: np.ndarray, dtype: str, device) -> torch.Tensor:
    """float32 array of bf16-representable values -> device tensor in ``dtype`` (exact)."""
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(arr_f32)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr_f32, dtype=np.float32)).to(device)


def _upload(w: Workload, layer: int, spec, dtype: str, device) -> torch.Tensor:
    name = spec[0]
    if is_matrix(name) and dtype == "bf16":
        bits = draw(w, layer, spec, "bf16")
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(draw(w, layer, spec, "f32")).to(device)


class DeviceModel:
    """All weights of a workload on the GPU plus the ``wam_weights`` struct pointing at them."""

    PACKED_MATS = ("w_qkv", "w_o", "w_cq", "w_co", "w_ff1", "w_ff2")

    def __init__(self, w: Workload, dtype: str = "bf16", device="cuda:0", overrides=None, packed=False):
        """packed: give every block its fragment-packed projections (bf16, native precision) and drop the
        unpacked copies of those six matrices, so only the packed ones can be read."""
        self.w, self.dtype, self.device = w, dtype, torch.device(device)
        self.cfg = make_config(w, dtype)
        self.packed = bool(packed)
        if self.packed and (dtype != "bf16" or self.cfg.precision != 0):
            raise ValueError("packed projections need dtype bf16 and native precision")
        overrides = overrides or {}
        self.g = {}
        for spec in global_tensors(w):
            self.g[spec[0]] = self._get(-1, spec, overrides)
        self.layers = []
        for l in range(w.layers):
            self.layers.append({spec[0]: self._get(l, spec, overrides) for spec in layer_tensors(w)})
        self._build_structs()

    def _get(self, layer, spec, overrides):
        key = (layer, spec[0])
        if key in overrides:
            arr = np.ascontiguousarray(overrides[key], dtype=np.float32)
            if is_matrix(spec[0]):
                return to_device(arr, self.dtype, self.device)
            return torch.from_numpy(arr).to(self.device)
        return _upload(self.w, layer, spec, self.dtype, self.device)

    def _build_structs(self):
        # The library reads matrices in the model dtype and every other tensor as float32.
        want = torch_dtype(self.dtype)
        for name, t in list(self.g.items()) + [kv for lp in self.layers for kv in lp.items()]:
            expect = want if is_matrix(name) else torch.float32
            if t.dtype != expect or not t.is_contiguous():
                raise TypeError("%s: %s (contiguous=%s), the library expects %s" % (name, t.dtype, t.is_contiguous(), expect))
        self.blocks = (wam_block_weights * self.w.layers)()
        for l, lp in enumerate(self.layers):
            for name, t in lp.items():
                setattr(self.blocks[l], name, t.data_ptr())
        self.mx = []
        if self.cfg.precision != 0:   # MXFP8 / MXFP4 weights: the library packs each layer's projections once
            nbytes = wam_mx_block_bytes(self.cfg)
            if nbytes == 0:
                raise ValueError("configuration cannot take MXFP8 projections")
            for l in range(self.w.layers):
                buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
                off = (-buf.data_ptr()) % 256
                arena = buf[off:off + nbytes]
                wam_mx_pack_block(self.cfg, self.blocks[l], arena)
                self.blocks[l].mx = arena.data_ptr()
                self.mx.append(buf)
        self.pk = []
        if self.packed:   # the library packs each layer's six projections once; the unpacked ones go
            nbytes = wam_pack_block_bytes(self.cfg)
            if nbytes == 0:
                raise ValueError("configuration cannot take packed projections")
            for l in range(self.w.layers):
                buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
                off = (-buf.data_ptr()) % 256
                arena = buf[off:off + nbytes]
                wam_pack_block(self.cfg, self.blocks[l], arena)
                self.blocks[l].pk = arena.data_ptr()
                self.pk.append(buf)
            torch.cuda.synchronize(self.device)
            for l, lp in enumerate(self.layers):
                for name in self.PACKED_MATS:
                    del lp[name]
                    setattr(self.blocks[l], name, None)
        self.weights = wam_weights()
        self.weights.blocks = ctypes.cast(self.blocks, ctypes.POINTER(wam_block_weights))
        for name in GLOBAL_FIELDS:
            t = self.g.get(name)
            setattr(self.weights, name, t.data_ptr() if t is not None else None)
        for name in ("st_w", "st_b"):
            t = self.g.get(name)
            setattr(self.weights, name, t.data_ptr() if t is not None else None)
        E = self.w.embodiments
        self.embodiments = (wam_action_io * E)()
        for e in range(E):
            suffix = "" if e == 0 else "_%d" % e
            for name in ("ae_w", "ae_b", "ao_w", "ao_b"):
                setattr(self.embodiments[e], name, self.g[name + suffix].data_ptr())
        self.weights.embodiments = ctypes.cast(self.embodiments, ctypes.POINTER(wam_action_io))
        self.weights.n_embodiments = E

    def for_embodiment(self, e: int) -> wam_weights:
        """The weights routed to embodiment e (its action encoder and decoder), as the library builds them."""
        return wam_weights_for_embodiment(self.weights, e)


class DeviceCache:
    """Self-attention KV cache [layers][br][heads][cap][d] (keys) / [..][d][cap] (values)."""

    def __init__(self, w: Workload, capacity: int, dtype: str = "bf16", device="cuda:0", branches=None):
        br = branches if branches is not None else w.branches
        cap = (capacity + 63) // 64 * 64
        td = torch_dtype(dtype)
        self.k = torch.zeros((w.layers, br, w.heads, cap, w.head_dim), dtype=td, device=device)
        self.v = torch.zeros((w.layers, br, w.heads, w.head_dim, cap), dtype=td, device=device)
        self.c = wam_kv_cache(self.k.data_ptr(), self.v.data_ptr(), br, cap, 0)

    @property
    def length(self) -> int:
        return self.c.length


class DeviceCtx:
    """Cross-attention keys/values of the condition sequence for every layer."""

    def __init__(self, w: Workload, dtype: str = "bf16", device="cuda:0", branches=None):
        br = branches if branches is not None else w.branches
        Lc = w.ctx_len
        stride = (Lc + 63) // 64 * 64
        td = torch_dtype(dtype)
        self.k = torch.zeros((w.layers, br, w.heads, Lc, w.head_dim), dtype=td, device=device)
        self.v = torch.zeros((w.layers, br, w.heads, w.head_dim, stride), dtype=td, device=device)
        self.c = wam_ctx_kv(self.k.data_ptr(), self.v.data_ptr(), br, Lc, stride)


def workspace(cfg: wam_config, n_chunks: int, device="cuda:0") -> torch.Tensor:
    nbytes = wam_workspace_bytes(cfg, n_chunks)
    if nbytes == 0:
        raise ValueError("invalid configuration for a workspace")
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]
