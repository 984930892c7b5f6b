"""Seeded synthetic inputs shared, as data only, by the CPU oracle and the HIP path.

Nothing here computes any step of the denoising method. The module turns
(base seed, workload, layer, tensor name) into a 64-bit key and fills arrays
from a Philox4x32-10 counter stream (see ``synth.c`` for the exact recipe).
Values are bfloat16-representable, returned either as raw bf16 bits
(``uint16``) or as the same values in ``float32``.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "_synth.so")
_lib = None
_lock = threading.Lock()

BASE_SEED = 1140  # the seed the inference examples on the pages use

_M64 = (1 << 64) - 1


def build(force: bool = True) -> str:
    """Compile ``synth.c`` into ``_synth.so`` with gcc (OpenMP, -O3)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC", _SRC, "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            lib.synth_fill.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
            lib.synth_fill.restype = None
            lib.synth_philox.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            lib.synth_philox.restype = None
            lib.synth_bf16_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64]
            lib.synth_f32_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64]
            lib.synth_uniform01_f64.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p]
            _lib = lib
    return _lib


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def _fnv1a64(s: str) -> int:
    h = 0xCBF29CE484222325
    for b in s.encode():
        h ^= b
        h = (h * 0x100000001B3) & _M64
    return h


def tensor_key(workload: int, layer: int, name: str, seed: int = BASE_SEED) -> int:
    """64-bit Philox key of one tensor: a splitmix64 chain over its identity."""
    k = _splitmix64(seed & _M64)
    k = _splitmix64(k ^ (workload & _M64))
    k = _splitmix64(k ^ ((layer + 1) & _M64))
    k = _splitmix64(k ^ _fnv1a64(name))
    return k


def philox4x32_10(ctr, key):
    """Raw Philox4x32-10 block (for the generator's known-answer test)."""
    lib = _load()
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib.synth_philox(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def normal_scale(sigma: float) -> np.float32:
    """fp32 factor that maps the centred Irwin-Hall(8) integer to std ``sigma``."""
    return np.float32(sigma / (2.0 * math.sqrt(8.0 * (65536.0 ** 2 - 1.0) / 12.0)))


def fill(shape, key: int, kind: str = "normal", sigma: float = 0.02, fmt: str = "f32", stream: int = 0):
    """Return an array of ``shape`` filled from the keyed stream.

    kind: "normal" (mean 0, std ``sigma``) or "uniform" ([-1, 1)).
    fmt:  "f32" (float32 values), "bf16" (uint16 bf16 bits) or "both".
    """
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    kind_i = 0 if kind == "normal" else 1
    c = normal_scale(sigma) if kind_i == 0 else np.float32(0.0)
    b = np.empty(shape, dtype=np.uint16) if fmt in ("bf16", "both") else None
    f = np.empty(shape, dtype=np.float32) if fmt in ("f32", "both") else None
    if n:
        lib.synth_fill(ctypes.c_uint64(key), ctypes.c_uint32(stream), kind_i, ctypes.c_float(float(c)),
                       ctypes.c_uint64(n), b.ctypes.data if b is not None else None,
                       f.ctypes.data if f is not None else None)
    if fmt == "both":
        return b, f
    return b if fmt == "bf16" else f


def constant(shape, value: float, fmt: str = "f32"):
    f = np.full(shape, value, dtype=np.float32)
    if fmt == "f32":
        return f
    b = f32_to_bf16_bits(f)
    return b if fmt == "bf16" else (b, f)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even), returned as uint16 bits."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.size:
        lib.synth_f32_to_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def uniform01(n: int, key: int, stream: int = 1) -> np.ndarray:
    """n host doubles in [0, 1) with 53 random bits each; used for timesteps."""
    lib = _load()
    out = np.empty(n, dtype=np.float64)
    if n:
        lib.synth_uniform01_f64(ctypes.c_uint64(key), ctypes.c_uint32(stream), ctypes.c_uint64(n), out.ctypes.data)
    return out


from .workloads import WORKLOADS, Workload, layer_tensors, global_tensors, input_tensors  # noqa: E402,F401
