"""CPU oracle of one denoising step of DreamZero's chunk-causal video+action DiT.

TEST INFRASTRUCTURE ONLY. The oracle is imported, called or run only by
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``. The product path (the HIP library and its binding) never
imports it, and the oracle never imports the product path: the two share
nothing but the seeded inputs drawn by the ``synth`` package.

Parity status: every function here is pinned by a CPU test against something
other than itself (closed forms, library routines, invariants the pages fix,
brute force on tiny shapes), except the composition with DreamZero's trained
weights, which is *parity unpinned*: no checkpoint and no worked numerical
example exist on the pages.
"""
from .dit import *  # noqa: F401,F403
from .unipc import denoise_chunk_unipc, exp_neg_h, step_order, update_weights  # noqa: F401
from .mx import (e2m1_encode, e2m1_value, e4m3_encode, e4m3_value, mx_attention, mx_dequantize, mx_linear,  # noqa: F401
                 mx_quantize, relative_error_bound, round_bf16)  # noqa: F401
