"""The allocation-free flow step (wam_flow_step_noalloc, cosine partials in the library's device
scratch) against wam_flow_step with a caller workspace, through the C ABI: two calls in a row, the
second on a smaller latent, each bit-identical to the workspace entry point on the same inputs (same
kernels, same grid for the same sizes, so the same summation order)."""
import numpy as np
import pytest
import torch

import synth
import world_action_video_amd as wam

pytestmark = pytest.mark.gpu


def _inputs(nv, na, seed):
    key = synth.tensor_key(102, seed, "noalloc-flow")
    v = synth.fill((2, nv + na), key, "normal", 1.0)
    x = synth.fill((nv + na,), key + 1, "normal", 1.0)
    prev = synth.fill((nv,), key + 2, "normal", 1.0)
    return x, v, prev


def _run(gpu, nv, na, x, v, prev, noalloc):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(gpu)  # noqa: E731
    xv, xa = d(x[:nv]), d(x[nv:])
    vv, va = d(v[:, :nv]), d(v[:, nv:])
    gv, ga = torch.full((nv,), float("nan"), device=gpu), torch.full((na,), float("nan"), device=gpu)
    cos = torch.full((3,), float("nan"), device=gpu)
    args = (xv, xa, vv, va, 2, 5.0, nv, na, 1.0 / 16, 0.25, gv, ga, d(prev), cos)
    if noalloc:
        wam.wam_flow_step_noalloc(*args)
    else:
        ws = torch.empty(8192, dtype=torch.uint8, device=gpu)
        wam.wam_flow_step(*args, ws)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (xv, xa, gv, ga, cos)]


def test_flow_step_noalloc_matches_workspace_call(gpu):
    # first call: 512 workgroups (the whole scratch), vector path; second: 8 workgroups, ragged sizes
    # (scalar path), so stale partials of the first call sit past the ones the second call reads
    for nv, na, seed in ((3_000_000, 4096, 0), (28161, 193, 1)):
        print("noalloc flow step", nv, na, flush=True)
        x, v, prev = _inputs(nv, na, seed)
        ref = _run(gpu, nv, na, x, v, prev, noalloc=False)
        got = _run(gpu, nv, na, x, v, prev, noalloc=True)
        for r, g in zip(ref, got):
            assert np.isfinite(g).all()
            assert np.array_equal(r, g)
        # and the step did run: x moved by dt times the guided velocity, the cosine terms are sums
        g_ref = 5.0 * v[0, :nv] - 4.0 * v[1, :nv]
        np.testing.assert_allclose(got[2], g_ref, rtol=1e-6, atol=1e-5)
        g64, p64 = g_ref.astype(np.float64), prev.astype(np.float64)
        exact = [g64 @ p64, g64 @ g64, p64 @ p64]
        scale = [np.abs(g64) @ np.abs(p64), exact[1], exact[2]]
        assert all(abs(float(c) - e) <= 1e-4 * s for c, e, s in zip(got[4], exact, scale))
