"""Benchmark: one flow-matching denoising step of the 40-layer chunk-causal DiT, CFG as a batch of 2.

Workload (Wan2.1-14B-shaped, synthetic): width 5120, 40 heads of 128, FFN 13824, 40 layers; one chunk
of 2 latent frames x 11 x 20 patches + 24 action tokens (464 tokens) per branch, 2 branches
(conditional / negative prompt); KV cache of 2 clean chunks (928 tokens); 769 condition tokens
(512 text + 257 image). A step = time-embedding MLP -> token embedding -> 40 blocks -> output heads ->
CFG + Euler + cosine partials, i.e. every kernel of the per-step path. The condition keys/values and
the cached chunks are built once before timing (they are per request, not per step).

Prints one JSON line (see the keys below). --gpus N > 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the MXFP8 scaled instructions run at this rate)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
WORKLOAD_ID = 3


def step_flops(w) -> dict:
    """Algorithmic FLOPs of one step (2*M*N*K per product; attention 4*br*H*Lq*Lk*d per self/cross)."""
    br, D, F, L, H, d = w.branches, w.dim, w.ffn_dim, w.layers, w.heads, w.head_dim
    Lq = w.chunk_tokens
    M = br * Lq
    Lk = w.cache_chunks * Lq + Lq
    gemm_layer = 2 * M * D * (3 * D + D + D + D + F + F)          # qkv, o, cross-q, cross-o, ffn1, ffn2
    attn_layer = 4 * br * H * Lq * d * (Lk + w.ctx_len)
    head = 2 * br * (w.video_tokens * D * w.patch_dim + w.action_tokens * D * w.action_dim)
    time_mlp = 2 * 2 * (D * w.freq_dim + D * D + 6 * D * D)
    return {"gemm": L * gemm_layer, "attention": L * attn_layer, "other": head + time_mlp,
            "total": L * (gemm_layer + attn_layer) + head + time_mlp}


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_key: str, src_hash: str):
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or None when the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_key)
    except Exception:
        return None
    if not rec or rec.get("source_sha256_16") != src_hash:
        return None
    return rec.get("bytes_per_launch")


TRAFFIC_KEY = "gemm_qkv_bf16_928x15360x5120"


def summarize_counters(fetch_db: str, write_db: str):
    """HBM bytes per launch of the QKV product from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by the ratio of known bytes to counted bytes of the 1 GiB copy in the same run."""
    import sqlite3

    def per_dispatch(db, counter):
        if not os.path.isfile(db):
            raise SystemExit("no such database: %s" % db)
        cur = sqlite3.connect("file:%s?mode=ro" % db, uri=True).cursor()
        cols = [r[1] for r in cur.execute("pragma table_info(counters_collection)")]
        name_col = "kernel_name" if "kernel_name" in cols else "name"
        rows = cur.execute("select %s, counter_name, value from counters_collection" % name_col).fetchall()
        return [(n, v) for n, c, v in rows if c.startswith(counter)]

    out = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        rows = per_dispatch(db, counter)
        copy = max((v for n, v in rows if "elementwise" in n), default=None)
        gemm = [v for n, v in rows if "gemm4p_kernel<0" in n]
        if copy is None or not gemm:
            raise SystemExit("counters not found in %s" % db)
        known = float(1 << 30)   # the copy moves 2^28 floats each way
        out[counter] = {"copy_kib": copy, "factor": known / (copy * 1024.0), "gemm_kib_mean": sum(gemm) / len(gemm),
                        "gemm_launches": len(gemm)}
    fetch = out["FETCH_SIZE"]["gemm_kib_mean"] * 1024.0 * out["FETCH_SIZE"]["factor"]
    write = out["WRITE_SIZE"]["gemm_kib_mean"] * 1024.0 * out["WRITE_SIZE"]["factor"]
    rec = {"bytes_per_launch": fetch + write, "fetch_bytes": fetch, "write_bytes": write, "counters": out,
           "source_sha256_16": source_hash(os.path.join(ROOT, "world_action_video_amd", "csrc", "gemm.hip")),
           "commands": ["rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o run -- python bench.py --counters",
                        "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o run -- python bench.py --counters",
                        "python bench.py --summarize-counters <fetch db> <write db>"]}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[TRAFFIC_KEY] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps({TRAFFIC_KEY: {"bytes_per_launch": rec["bytes_per_launch"]}}))


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def measured_mfma_peak(wam, torch, dev):
    """bf16 TFLOP/s of back-to-back independent 32x32x16 MFMAs on every SIMD (the library's probe
    kernel, 256 workgroups of one wave per SIMD), median of 5 timed launches of about 1 ms."""
    wg, iters = 256, 4096
    out = torch.empty(wg * 256, device=dev)
    wam.wam_mfma_peak_probe(out, wg, iters)
    times = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        wam.wam_mfma_peak_probe(out, wg, iters)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    flops = wg * 4.0 * iters * 8 * 32768
    return round(flops / (median(times) * 1e-3) / 1e12, 1)


def host_description() -> dict:
    """CPU model and the BLAS NumPy runs on (vendor, version, threads)."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas.append({"vendor": i.get("internal_api"), "version": i.get("version"),
                             "threads": i.get("num_threads")})
    except Exception:
        pass
    return {"cpu_model": model, "blas": blas}


def short_kernel_name(n: str) -> str:
    """`wam::gemm4_kernel<0>` from the demangled signature of a kernel dispatch."""
    n = n.replace("void ", "").replace("(anonymous namespace)::", "")
    cut = n.find("(")
    return n[:cut] if cut > 0 else n


def summarize_trace(db: str):
    """Kernel trace of a bench.py run (rocprofv3 --kernel-trace): per-kernel totals, the wall time of
    each stack pass (between consecutive time-MLP launches), and one layer of the last timed step
    (the dispatches from the middle layer's QKV product to the next one). Markdown on stdout."""
    import sqlite3
    if not os.path.isfile(db):
        raise SystemExit("no such database: %s" % db)
    cur = sqlite3.connect("file:%s?mode=ro" % db, uri=True).cursor()
    rows = cur.execute("select name, start, end from kernels order by start").fetchall()
    ks = [(short_kernel_name(n), s0, e0) for n, s0, e0 in rows]
    tot = {}
    for n, s0, e0 in ks:
        c, t = tot.get(n, (0, 0.0))
        tot[n] = (c + 1, t + (e0 - s0) / 1e3)
    all_us = sum(t for _, t in tot.values())
    print("| kernel | calls | total (us) | average (us) | share |\n|---|---:|---:|---:|---:|")
    for n, (c, t) in sorted(tot.items(), key=lambda x: -x[1][1])[:20]:
        print("| `%s` | %d | %.1f | %.2f | %.1f%% |" % (n, c, t, t / c, 100 * t / all_us))
    starts = [s0 for n, s0, _ in ks if "sinusoid" in n]
    if len(starts) > 1:
        print("\nstack passes, wall time between consecutive time-embedding launches (ms): " +
              ", ".join("%.3f" % ((b - a) / 1e6) for a, b in zip(starts, starts[1:])))
    last = [i for i, (n, _, _) in enumerate(ks) if "sinusoid" in n]
    if len(last) >= 2:
        lo, hi = last[-2], last[-1]
        qkv = [i for i in range(lo, hi) if re.search(r"gemm4p?_kernel<0(>|, )", ks[i][0])]
        if len(qkv) > 21:
            a, b = qkv[20], qkv[21]
            print("\none layer of the last full stack pass (dispatch order, from the middle layer's QKV product):\n")
            print("| kernel | us |\n|---|---:|")
            for n, s0, e0 in ks[a:b]:
                print("| `%s` | %.1f |" % (n, (e0 - s0) / 1e3))
            print("| **layer (sum of kernel times)** | **%.1f** |" % (sum((e0 - s0) for _, s0, e0 in ks[a:b]) / 1e3))
            print("| layer wall time (QKV start to next QKV start) | %.1f |" % ((ks[b][1] - ks[a][1]) / 1e3))


def summarize_grid(db: str, name_filter: str):
    """Kernel durations of a rocprofv3 --kernel-trace database grouped by kernel and grid size (one
    line per launch shape: calls, median and minimum microseconds), for kernels whose name contains
    ``name_filter``. Markdown on stdout."""
    import sqlite3
    if not os.path.isfile(db):
        raise SystemExit("no such database: %s" % db)
    cur = sqlite3.connect("file:%s?mode=ro" % db, uri=True).cursor()
    groups = {}
    for n, gx, wx, s0, e0 in cur.execute("select name, grid_x, workgroup_x, start, end from kernels"):
        k = short_kernel_name(n)
        if name_filter in k:
            groups.setdefault((k, gx // max(wx, 1), wx), []).append((e0 - s0) / 1e3)
    print("| kernel | workgroups | threads | calls | median (us) | min (us) |\n|---|---:|---:|---:|---:|---:|")
    for (k, wgs, wx), ds in sorted(groups.items()):
        print("| `%s` | %d | %d | %d | %.2f | %.2f |" % (k, wgs, wx, len(ds), median(ds), min(ds)))


def summarize_pmc(dbs, name_filter: str):
    """Mean of every counter per dispatch, per kernel whose name contains ``name_filter``, over the
    rocprofv3 --pmc databases ``dbs`` (one pass each): a markdown table on stdout."""
    import sqlite3
    rows = {}
    for db in dbs:
        if not os.path.isfile(db):
            raise SystemExit("no such database: %s" % db)
        cur = sqlite3.connect("file:%s?mode=ro" % db, uri=True).cursor()
        cols = [r[1] for r in cur.execute("pragma table_info(counters_collection)")]
        name_col = "kernel_name" if "kernel_name" in cols else "name"
        for n, c, v in cur.execute("select %s, counter_name, value from counters_collection" % name_col):
            if name_filter in n:
                rows.setdefault(n, {}).setdefault(c, []).append(float(v))
    for n, cs in sorted(rows.items()):
        print("\n`%s`\n\n| counter | dispatches | mean per dispatch |\n|---|---:|---:|" % n)
        for c, vs in sorted(cs.items()):
            print("| %s | %d | %.4g |" % (c, len(vs), sum(vs) / len(vs)))


def cpu_baseline(w, timed_layers: int = 1) -> dict:
    """The oracle as it stands, timed on this host on a bounded sample: ``timed_layers`` full-width
    blocks of the workload's step (both CFG branches, its cached, current and condition tokens),
    scaled to ms per step of all its layers."""
    import numpy as np
    import oracle as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    m = O.load_model(w, layers=list(range(timed_layers)))
    Lq, D = w.chunk_tokens, w.dim
    T = Lq
    br = w.branches
    key = synth.tensor_key(w.id, -1, "cpu-baseline")
    h = synth.fill((br, T, D), key, "normal", 1.0)
    ctx_k = synth.fill((br, w.ctx_len, D), key + 1, "normal", 1.0)
    ctx_v = synth.fill((br, w.ctx_len, D), key + 2, "normal", 1.0)
    ck = synth.fill((br, w.cache_chunks * Lq, D), key + 3, "normal", 1.0)
    cv = synth.fill((br, w.cache_chunks * Lq, D), key + 4, "normal", 1.0)
    e6, _ = O.per_token_time(w, m.g, [0.5], [0.5], 1, np.float32)
    pos = O.video_positions(w, 1, w.cache_chunks * w.frames_per_chunk)
    t0 = time.perf_counter()
    for lp in m.layers:
        h, _, _ = O.block_forward(w, lp, h, e6, ctx_k, ctx_v, ck, cv, 1, pos)
    dt = time.perf_counter() - t0
    per_layer = dt / timed_layers
    return {**host_description(), "value": round(per_layer * w.layers * 1e3, 1),
            "unit": "ms per %d-layer CFG step (extrapolated)" % w.layers if w.layers > 1 else "ms per block",
            "cores": int(threads), "kind": "oracle",
            "sample": "%d full-width block(s) of the step (CFG batch %d, %d cached + %d current tokens, %d "
                      "condition tokens), NumPy fp32, %.2f s per block, scaled x%d layers; time MLP and heads "
                      "(<0.1%% of FLOPs) not timed" % (timed_layers, br, w.cache_chunks * Lq, Lq, w.ctx_len,
                                                       per_layer, w.layers)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=WORKLOAD_ID, choices=(2, 3, 4, 5),
                    help="3: the step metric (default); 2: one full-width block (br = 2 and B = 1); 4: four chunks "
                         "of 16 Euler steps plus KV appends; 5: three-view long context, 16-step loop with reuse")
    ap.add_argument("--unpacked", action="store_true",
                    help="bf16 projections from the unpacked [out][in] matrices instead of the fragment-packed copies "
                         "(the default); for comparisons on one box, reported under its own workload name")
    ap.add_argument("--precision", choices=("bf16", "mxfp8", "mxfp4w"), default="bf16",
                    help="bf16 (the metric); mxfp8: the six block projections quantised to MXFP8; mxfp4w: their "
                         "weights MXFP4, activations MXFP8 -- reported separately (own dtype and workload name)")
    ap.add_argument("--variant", type=int, default=0,
                    help="architectural variant bits of the step (1 frame-causal, 2 RMSNorm, 4 SwiGLU, 8 separate "
                         "image cross-attention); non-zero values are reported under their own workload name")
    ap.add_argument("--counters", action="store_true",
                    help="run only a 1 GiB copy and launches of the dominant kernel (for rocprofv3 --pmc)")
    ap.add_argument("--elementwise", action="store_true",
                    help="HBM-bound kernels: the flow update from the step's size to a >1 GB footprint (buffers "
                         "rotated through a 1.5 GiB pool, past the 256 MB Infinity Cache) beside a 1 GiB copy, and one "
                         "one full-width block of the 40-layer step over 1 and 8 chunks (for a kernel trace of its row kernels)")
    ap.add_argument("--attention", action="store_true",
                    help="bf16 and MXFP8 attention kernels at the step's self- and cross-attention shapes")
    ap.add_argument("--attention-shape", choices=("self", "cross", "both"), default="both",
                    help="with --attention: only the self- or only the cross-attention shape (one shape per counter run)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DB",
                    help="per-kernel mean of every counter in rocprofv3 --pmc databases (kernels whose name contains "
                         "--kernel-filter)")
    ap.add_argument("--kernel-filter", default="", help="substring of the kernel names --summarize-pmc reports")
    ap.add_argument("--summarize-grid", metavar="DB",
                    help="kernel durations of a rocprofv3 --kernel-trace database per kernel and grid size "
                         "(with --kernel-filter)")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="per-kernel totals, stack-pass wall times and one layer's dispatches of a rocprofv3 "
                         "--kernel-trace database of a bench.py run")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="turn the two rocprofv3 --pmc databases of a --counters run (FETCH_SIZE, WRITE_SIZE) "
                         "into profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.summarize_grid:
        summarize_grid(args.summarize_grid, args.kernel_filter)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.kernel_filter)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print("bench.py: this path runs on one GPU; --gpus %d is not supported (run with --gpus 1)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import world_action_video_amd as wam
    from synth.workloads import WORKLOADS, draw_named
    from world_action_video_amd.device import DeviceCache, DeviceCtx, DeviceModel, to_device, workspace

    dev = torch.device("cuda:0")
    if args.elementwise:
        elementwise(args, dev)
        return
    if args.attention:
        attention_kernels(args, dev)
        return
    if args.workload != WORKLOAD_ID and not args.counters:
        extra_workload(args, dev)
        return
    w = WORKLOADS[WORKLOAD_ID]
    mx = args.precision != "bf16"
    w4 = args.precision == "mxfp4w"
    if mx:
        w = w.with_(precision=synth.workloads.PRECISION_MXFP4W if w4 else synth.workloads.PRECISION_MXFP8)
    if args.variant:
        w = w.with_(variant=args.variant)
    Lq, Lv, La, D = w.chunk_tokens, w.video_tokens, w.action_tokens, w.dim
    M = w.branches * Lq

    if args.counters:
        # calibration copy (known bytes) and launches of the dominant kernel at the step's shape
        x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.mul(x, 1.0, out=y)
        a = torch.randn((M, D), device=dev).to(torch.bfloat16)
        wq = (torch.randn((3 * D, D), device=dev) * 0.02).to(torch.bfloat16)
        wqp = torch.empty_like(wq)
        wam.wam_pack_weight(wq, D, 3 * D, D, wqp)
        c = torch.empty((M, 3 * D), dtype=torch.bfloat16, device=dev)
        for _ in range(5):
            wam.wam_op_linear_packed(a, D, wqp, None, c, 3 * D, M, 3 * D, D, 0)
        torch.cuda.synchronize()
        print(json.dumps({"counters_run": True, "copy_bytes_read": x.numel() * 4, "copy_bytes_written": y.numel() * 4}))
        return

    def log(msg):
        print("[bench] %s" % msg, file=sys.stderr, flush=True)

    t_setup = time.perf_counter()
    packed = not mx and not args.unpacked
    log("uploading %s weights%s" % (w.name, " (fragment-packed projections)" if packed else ""))
    model = DeviceModel(w, "bf16", dev, packed=packed)
    log("weights resident (%.1f s); building condition KV and %d cached chunks" % (time.perf_counter() - t_setup,
                                                                                  w.cache_chunks))
    ws = workspace(model.cfg, 1, dev)
    ctx = DeviceCtx(w, "bf16", dev)
    txt = draw_named(w, -1, "txt")
    img = draw_named(w, -1, "img")
    wam.wam_ctx_build(model.cfg, model.weights, to_device(txt, "bf16", dev), to_device(img, "bf16", dev), ctx.c, ws)
    cache = DeviceCache(w, (w.cache_chunks + 1) * Lq, "bf16", dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)  # noqa: E731
    for c in range(w.cache_chunks):
        wam.wam_kv_append(model.cfg, model.weights, cache.c, ctx.c, f32(draw_named(w, -1, "x1_video_%d" % c)),
                          f32(draw_named(w, -1, "x1_action_%d" % c)), c * w.frames_per_chunk, ws)
    assert cache.length == w.cache_chunks * Lq
    start_frame = w.cache_chunks * w.frames_per_chunk
    xv = f32(draw_named(w, -1, "eps_video_%d" % w.cache_chunks))
    xa = f32(draw_named(w, -1, "eps_action_%d" % w.cache_chunks))
    vv = torch.empty((w.branches, Lv, w.patch_dim), device=dev)
    va = torch.empty((w.branches, La, w.action_dim), device=dev)
    gv = torch.zeros(Lv * w.patch_dim, device=dev)
    ga = torch.zeros(La * w.action_dim, device=dev)
    cos = torch.zeros(3, device=dev)
    fws = torch.empty(4096, dtype=torch.uint8, device=dev)
    ts = synth.workloads.timesteps(w, args.steps + args.warmup)
    nv, na = Lv * w.patch_dim, La * w.action_dim
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def step(t):
        wam.wam_dit_stack_fwd(model.cfg, model.weights, cache.c, ctx.c, 1, xv, xa, [t], [t], start_frame, vv, va, ws)
        wam.wam_flow_step(xv, xa, vv, va, w.branches, w.guidance, nv, na, 1.0 / 16, 1.0 / 16, gv, ga, gv, cos, fws)

    log("setup done (%.1f s); warmup %d, timed %d steps" % (setup_s, args.warmup, args.steps))
    t_first = time.perf_counter()
    step(float(ts[0]))
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t_first) * 1e3
    for i in range(1, args.warmup):
        step(float(ts[i]))
    torch.cuda.synchronize()
    # the dominant kernel is timed inside the timed steps: one event pair per step around the QKV
    # product of the middle layer, recorded by the library on its own stream
    timer_layer = w.layers // 2
    wam.wam_qkv_timer_config(timer_layer, args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]   # one boundary per step
    evs[0].record()
    for i in range(args.steps):
        step(float(ts[args.warmup + i]))
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    step_samples = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    qkv_samples = wam.wam_qkv_timer_read(args.steps)
    wam.wam_qkv_timer_config(-1)
    finite = bool(torch.isfinite(vv).all().item() and torch.isfinite(va).all().item())

    # dominant kernel: the QKV projection GEMM (M = 928, N = 15360, K = 5120; bf16 MFMA on the fragment-packed
    # weights, or the scaled fp8 MFMA on the MX-packed ones). The roofline uses the in-step samples above; 20
    # back-to-back launches of the same kernel and launch configuration (layer 0's weights, HIP events on the
    # library's stream) are reported beside them: they run at the lower clock of sustained matrix work
    y = torch.randn((M, D), device=dev).to(torch.bfloat16)
    cq = torch.empty((M, 3 * D), dtype=torch.bfloat16, device=dev)
    bq = model.layers[0]["b_qkv"]
    if packed:   # w_qkv's packed copy opens layer 0's arena
        qkv_op = lambda: wam.wam_op_linear_packed(y, D, model.blocks[0].pk, bq, cq, 3 * D, M, 3 * D, D, 0)  # noqa: E731
    elif mx:
        yq = torch.empty((M, D), dtype=torch.uint8, device=dev)
        ys = torch.empty((M, D // 32), dtype=torch.uint8, device=dev)
        wam.wam_mx_quantize(wam.WAM_BF16, y, D, M, D, yq, D, ys)
        arena = model.blocks[0].mx   # w_qkv codes [3D][D] (or [3D][D/2] packed e2m1) at 0, its scales after them
        wrow = D // 2 if w4 else D
        wq_s = arena + ((3 * D * wrow + 255) // 256) * 256
        qkv_op = lambda: wam.wam_op_linear_mx(yq, ys, D, arena, wq_s, wrow, bq, cq, 3 * D, M, 3 * D, D, 0,  # noqa: E731
                                              w_format=wam.WAM_MX_E2M1 if w4 else wam.WAM_MX_E4M3)
    else:
        wq = model.layers[0]["w_qkv"]
        qkv_op = lambda: wam.wam_op_linear(wam.WAM_BF16, y, D, wq, D, bq, cq, 3 * D, M, 3 * D, D, 0)  # noqa: E731
    for _ in range(3):
        qkv_op()
    reps = 20
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        qkv_op()
    e1.record()
    torch.cuda.synchronize()
    b2b_ms = e0.elapsed_time(e1) / reps
    gemm_mean_ms = sum(qkv_samples) / len(qkv_samples) if qkv_samples else b2b_ms
    gemm_ms = median(qkv_samples) if qkv_samples else b2b_ms
    peak_meas = measured_mfma_peak(wam, torch, dev)
    gemm_flops = 2.0 * M * 3 * D * D
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    traffic = None if not packed else load_traffic(TRAFFIC_KEY, source_hash(os.path.join(ROOT, "world_action_video_amd",
                                                                                          "csrc", "gemm.hip")))
    peak = PEAK_FP8_TFLOPS if mx else PEAK_BF16_TFLOPS

    fl = step_flops(w)
    step_tflops = fl["total"] / (ms * 1e-3) / 1e12
    out = {
        "metric": "ms per DiT denoise step (40L, CFG b=2)",
        "value": round(ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("mxfp4 weights x mxfp8 activations in the projections, bf16 elsewhere" if w4 else
                  "mxfp8 projections, bf16 elsewhere") if mx else "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) latents/features)",
        "config": {"workload": w.name + (("+mxfp4w-projections" if w4 else "+mxfp8-projections") if mx else "") +
                               ("+unpacked-weights" if args.unpacked and not mx else "") +
                               ("+variant%d" % args.variant if args.variant else ""), "layers": w.layers, "dim": w.dim, "heads": w.heads, "head_dim": w.head_dim,
                   "ffn_dim": w.ffn_dim, "branches": w.branches, "chunk_tokens": Lq, "cached_tokens": cache.length,
                   "ctx_tokens": w.ctx_len},
        "step_tflop": round(fl["total"] / 1e12, 3),
        "step_tflops": round(step_tflops, 1),
        "step_mfma_frac": round(step_tflops / PEAK_BF16_TFLOPS, 4),
        "median_ms": round(median(step_samples), 3),
        "min_ms": round(step_samples[0], 3),
        "max_ms": round(step_samples[-1], 3),
        "first_step_ms": round(first_ms, 1),
        "setup_s": round(setup_s, 1),
        "outputs_finite": finite,
        "roofline": {"kernel": ("gemm4mx_kernel<EPI_STORE, W4> (MXFP4 x MXFP8 scaled MFMA, 256x256 tile" if w4 else
                                "gemm4mx_kernel<EPI_STORE> (MXFP8 scaled MFMA, 256x256 tile" if mx else
                                "gemm4p_kernel<EPI_STORE, 5, 3> (bf16, fragment-packed weights, 160x384 tile, waves "
                                "side by side along N" if packed else
                                "gemm4_kernel<EPI_STORE, 3, 5> (bf16, 192x320 tile") + ", 4 waves; QKV projection, "
                                "928x15360x5120)",
                     "bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / peak, 4), "traffic": traffic,
                     "avg_launch_us": round(gemm_ms * 1e3, 2),
                     "mean_launch_us": round(gemm_mean_ms * 1e3, 2),
                     "timing": "median of HIP event pairs around layer %d's QKV launch in each of the %d timed steps "
                               "(%d samples; mean beside it)" % (timer_layer, args.steps, len(qkv_samples)),
                     "measured_peak_tflops": peak_meas,
                     "back_to_back_us": round(b2b_ms * 1e3, 2)},
    }
    log("step %.3f ms; QKV GEMM %.1f us (%.1f TFLOP/s)" % (ms, gemm_ms * 1e3, gemm_tflops))
    if not args.no_cpu_baseline and not mx and not args.variant:
        log("timing the oracle on the host")
        del model, cache, ctx
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out))


def elementwise(args, dev):
    """HBM-bound kernels at the step's size and past the Infinity Cache (one JSON line): the flow
    update, the split-K finish, the standalone adaLN and the q/k/v post-processing, each resident and
    rotated up to >= 1 GB per call, the 1 GiB device copy, and one block over 1 and 8 chunks.

    Flow update (guidance + Euler + cosine partials, 2 branches): 24 bytes per latent element (reads x,
    v_cond, v_uncond, prev; writes x, g). Guidance 1 and dt 0 keep every value bounded while the kernel
    still moves all of them. "resident" reuses one buffer set per call; "rotated" walks the calls through a
    1.5 GiB pool so that consecutive calls touch new memory. The copy is torch's device copy of 1 GiB
    between two rotated pairs (2 GiB moved per call), the practical HBM ceiling next to the 8 TB/s
    nominal figure. The block pass runs layer 0 of the 40-layer CFG-2 step (928 cached tokens) over 1 and 8 chunks: its split-K
    finishes and q/k/v kernel then see 105 MB and 840 MB footprints, timed per kernel by a trace."""
    import torch

    import world_action_video_amd as wam
    from synth.workloads import WORKLOADS, draw_named
    from world_action_video_amd.device import DeviceCache, DeviceCtx, DeviceModel, to_device, workspace

    def log(msg):
        print("[bench] %s" % msg, file=sys.stderr, flush=True)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(fn, reps):
        a, b = ev(), ev()
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    pool_floats = 384 << 20                                  # 1.5 GiB
    pool = torch.randn(pool_floats, device=dev)
    na = 192
    cos = torch.zeros(3, device=dev)
    fws = torch.empty(32768, dtype=torch.uint8, device=dev)
    flow = []
    for nv in (28160, 1 << 20, 1 << 22, 1 << 24, 50 << 20):
        n = nv + na
        span = (5 * n + 63) // 64 * 64                       # x, v (2 branches), prev, g
        sets = max(1, pool_floats // span)
        nbytes = 24 * n

        base = pool.data_ptr()

        def call(i, rot):
            # one set: x [nv | na], v [2][nv] then [2][na], prev [nv], g [nv | na] (raw pointers keep the
            # host side of a call short)
            o = base + 4 * ((i % sets) * span if rot else 0)
            x, v, pv, g = o, o + 4 * n, o + 12 * n, o + 16 * n
            wam.wam_flow_step(x, x + 4 * nv, v, v + 8 * nv, 2, 1.0, nv, na, 0.0, 0.0, g, g + 4 * nv, pv, cos, fws)

        reps = min(4000, max(20, 2 * sets)) if sets > 1 else 10
        for rot in (False, True):
            call(0, rot)
        res = timed(lambda i: call(i, False), 20 if nv > (1 << 22) else 200)
        rot = timed(lambda i: call(i, True), reps)
        flow.append({"n": n, "bytes": nbytes, "resident_us": round(res * 1e3, 2),
                     "resident_GBps": round(nbytes / (res * 1e-3) / 1e9, 1),
                     "rotated_us": round(rot * 1e3, 2), "rotated_GBps": round(nbytes / (rot * 1e-3) / 1e9, 1),
                     "rotated_hbm_frac": round(nbytes / (rot * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
        log("flow n=%d: resident %.2f us, rotated %.2f us (%.0f GB/s)" % (n, res * 1e3, rot * 1e3,
                                                                          nbytes / (rot * 1e-3) / 1e9))
    del pool
    torch.cuda.empty_cache()
    src = [torch.ones(1 << 28, device=dev) for _ in range(2)]
    dst = [torch.empty(1 << 28, device=dev) for _ in range(2)]
    dst[0].copy_(src[0])
    copy_ms = timed(lambda i: dst[i % 2].copy_(src[i % 2]), 20)
    copy_gbps = 2 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    log("copy 1 GiB: %.1f us, %.0f GB/s" % (copy_ms * 1e3, copy_gbps))
    del src, dst
    torch.cuda.empty_cache()

    # Row kernels on their own, resident and rotated through a 4 GiB pool: the split-K finish (three
    # fp32 partials and the residual read, the residual and the bf16 norm output written: 22 B per
    # element) and the standalone adaLN (fp32 row in, bf16 out: 6 B per element). Per-column vectors
    # (bias, modulation) are not counted.
    D = 5120
    pool_floats = 1 << 30
    pool = torch.empty(pool_floats, device=dev)
    pool.normal_()
    vec = lambda: (torch.randn((6, D), device=dev) * 0.1)  # noqa: E731
    e6v, mgv, mnv, biasv = vec(), vec(), vec(), torch.randn(D, device=dev) * 0.1
    rowk = {"finish": [], "norm": []}
    for kind, Ms in (("finish", (928, 2784, 9280)), ("norm", (928, 7424, 37120))):
        for M in Ms:
            n = M * D
            span = ((4 * n + n // 2 if kind == "finish" else n + n // 2) + 63) // 64 * 64   # floats per set
            sets = max(1, pool_floats // span)
            nbytes = (22 if kind == "finish" else 6) * n
            base = pool.data_ptr()

            def call(i, rot, kind=kind, M=M, n=n, span=span, sets=sets, base=base):
                o = base + 4 * ((i % sets) * span if rot else 0)
                if kind == "finish":   # part [3][M][D], h [M][D], y bf16 [M][D]
                    wam.wam_op_split_finish(o, 3, M, D, biasv, o + 12 * n, e6v, mgv, 5, mnv, 0, 1, o + 16 * n)
                else:                  # x [M][D], y bf16 [M][D]
                    wam.wam_op_modulated_norm(o, M, D, e6v, mnv, 0, 1, o + 4 * n)

            for rot in (False, True):
                call(0, rot)
            res = timed(lambda i: call(i, False), 50 if n < (1 << 24) else 10)
            rot = timed(lambda i: call(i, True), max(10, min(400, 4 * sets)))
            rowk[kind].append({"rows": M, "bytes": nbytes, "sets": sets, "resident_us": round(res * 1e3, 2),
                               "resident_GBps": round(nbytes / (res * 1e-3) / 1e9, 1),
                               "rotated_us": round(rot * 1e3, 2), "rotated_GBps": round(nbytes / (rot * 1e-3) / 1e9, 1),
                               "rotated_hbm_frac": round(nbytes / (rot * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
            log("%s rows=%d: resident %.2f us, rotated %.2f us (%.0f GB/s)" % (kind, M, res * 1e3, rot * 1e3,
                                                                             nbytes / (rot * 1e-3) / 1e9))
    # q/k norm + rotary + cache scatter (2 branches, 40 heads of 128): q, k, v bf16 read, q, k, v bf16
    # written, 12 B per element of a row's D columns
    H, dh, br = 40, 128, 2
    ang = torch.rand((8352, dh // 2), device=dev) * 6.2832
    rope = torch.stack([torch.cos(ang), torch.sin(ang)], dim=-1).contiguous()
    gq, gk = torch.ones(D, device=dev), torch.ones(D, device=dev)
    rowk["qkv"] = []
    for rows in (464, 3712, 8352):
        n = br * rows * D
        span = (3 * n + 63) // 64 * 64       # floats per set: qkv (6 B), q, k, v (2 B each) per element
        sets = max(1, pool_floats // span)
        nbytes = 12 * n
        base = pool.data_ptr()

        def call(i, rot, rows=rows, n=n, span=span, sets=sets, base=base):
            o = base + 4 * ((i % sets) * span if rot else 0)
            wam.wam_op_qkv_cache(o, br, rows, 464, 440, H, dh, gq, gk, 1e-6, rope, o + 6 * n, o + 8 * n, o + 10 * n,
                                 rows, 0)

        for rot in (False, True):
            call(0, rot)
        res = timed(lambda i: call(i, False), 50 if n < (1 << 24) else 10)
        rot = timed(lambda i: call(i, True), max(10, min(400, 4 * sets)))
        rowk["qkv"].append({"rows": br * rows, "bytes": nbytes, "sets": sets, "resident_us": round(res * 1e3, 2),
                            "resident_GBps": round(nbytes / (res * 1e-3) / 1e9, 1),
                            "rotated_us": round(rot * 1e3, 2), "rotated_GBps": round(nbytes / (rot * 1e-3) / 1e9, 1),
                            "rotated_hbm_frac": round(nbytes / (rot * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)})
        log("qkv rows=%d: resident %.2f us, rotated %.2f us (%.0f GB/s)" % (br * rows, res * 1e3, rot * 1e3,
                                                                          nbytes / (rot * 1e-3) / 1e9))
    del pool
    torch.cuda.empty_cache()

    w = WORKLOADS[WORKLOAD_ID].with_(layers=1)
    Lq = w.chunk_tokens
    model = DeviceModel(w, "bf16", dev, packed=True)
    ctx = DeviceCtx(w, "bf16", dev)
    blocks = {}
    n_max = 8
    ws = workspace(model.cfg, n_max, dev)
    img = draw_named(w, -1, "img")
    wam.wam_ctx_build(model.cfg, model.weights, to_device(draw_named(w, -1, "txt"), "bf16", dev),
                      to_device(img, "bf16", dev), ctx.c, ws)
    cache = DeviceCache(w, (w.cache_chunks + n_max) * Lq, "bf16", dev)
    f32 = lambda a: torch.from_numpy(a.astype("float32")).to(dev)  # noqa: E731
    for c in range(w.cache_chunks):
        wam.wam_kv_append(model.cfg, model.weights, cache.c, ctx.c, f32(draw_named(w, -1, "x1_video_%d" % c)),
                          f32(draw_named(w, -1, "x1_action_%d" % c)), c * w.frames_per_chunk, ws)
    for n_chunks in (1, n_max):
        h = torch.randn((w.branches, n_chunks * Lq, w.dim), device=dev)
        e = torch.empty((2 * n_chunks, w.dim), device=dev)
        e6 = torch.empty((2 * n_chunks, 6, w.dim), device=dev)
        wam.wam_time_embed(model.cfg, model.weights, [0.4] * (2 * n_chunks), e, e6, ws)
        run = lambda i: wam.wam_dit_block_fwd(model.cfg, model.blocks[0], 0, cache.c, ctx.c, h, e6, n_chunks,  # noqa
                                              w.cache_chunks * w.frames_per_chunk, ws)
        run(0)
        blocks["chunks_%d" % n_chunks] = round(timed(run, 3), 3)
        log("block over %d chunk(s): %.3f ms" % (n_chunks, blocks["chunks_%d" % n_chunks]))
    print(json.dumps({"metric": "HBM-bound kernels (flow update sweep, 1 GiB copy, block passes)",
                      "unit": "GB/s", "n_gpus": 1, "dtype": "f32", "data": "synthetic",
                      "config": {"workload": "flow update 2 branches, 24 B per element; split-K finish, 22 B per "
                                             "element; adaLN, 6 B; q/k/v post-processing, 12 B; width 5120; "
                                             "one block of the 40-layer step over 1 and 8 chunks"},
                      "hbm_peak_GBps": PEAK_HBM_GBS, "copy_1GiB_GBps": round(copy_gbps, 1),
                      "copy_frac": round(copy_gbps / PEAK_HBM_GBS, 3), "flow": flow, "split_finish": rowk["finish"],
                      "modulated_norm": rowk["norm"], "qkv_cache": rowk["qkv"], "block_ms": blocks}))


def attention_kernels(args, dev):
    """bf16 (`attn3_kernel`) and MXFP8 (`attn_mx_kernel`) attention at the 40-layer step's shapes: self-attention
    of 2 branches x 40 heads, 464 queries over 928 cached + 464 current keys (chunk-causal), and
    cross-attention over the 769 condition tokens. Operands are random (N(0, 1), quantised on the
    device for the MXFP8 op); HIP events around 20 back-to-back launches. Work: 4 br H Lq Lk_visible d."""
    import torch

    import world_action_video_amd as wam

    br, H, Lq, d = 2, 40, 464, 128
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    out = {}
    for name, kv_total, kv_base, chunk_q in (("self", 1392, 928, 464), ("cross", 769, 0, 0)):
        if args.attention_shape not in ("both", name):
            continue
        v_stride = (kv_total + 63) // 64 * 64
        q = torch.randn((br, H, Lq, d), device=dev).to(torch.bfloat16)
        k = torch.randn((br, H, kv_total, d), device=dev).to(torch.bfloat16)
        vt = torch.zeros((br, H, d, v_stride), device=dev, dtype=torch.bfloat16)
        vt[..., :kv_total] = torch.randn((br, H, d, kv_total), device=dev).to(torch.bfloat16)
        o = torch.empty((br * Lq, H * d), dtype=torch.bfloat16, device=dev)
        qc = torch.empty((br, H, Lq, d), dtype=torch.uint8, device=dev)
        qs = torch.empty((br, H, Lq, d // 32), dtype=torch.uint8, device=dev)
        kc = torch.empty((br, H, kv_total, d), dtype=torch.uint8, device=dev)
        ks = torch.empty((br, H, kv_total, d // 32), dtype=torch.uint8, device=dev)
        vc = torch.empty((br, H, d, v_stride), dtype=torch.uint8, device=dev)
        vs = torch.empty((br, H, d, v_stride // 32), dtype=torch.uint8, device=dev)
        wam.wam_mx_quantize(wam.WAM_BF16, q, d, br * H * Lq, d, qc, d, qs)
        wam.wam_mx_quantize(wam.WAM_BF16, k, d, br * H * kv_total, d, kc, d, ks)
        wam.wam_mx_quantize(wam.WAM_BF16, vt, v_stride, br * H * d, v_stride, vc, v_stride, vs)
        vs_bm = vs.transpose(2, 3).contiguous()      # block-major scales of V^T
        ops = {
            "bf16": lambda: wam.wam_op_attention(wam.WAM_BF16, q, k, vt, o, br, H, d, Lq, kv_total, v_stride,
                                                 kv_base, chunk_q, kv_total),
            "mxfp8": lambda: wam.wam_op_attention_mx(qc, qs, kc, ks, vc, vs_bm, o, br, H, Lq, kv_total, v_stride,
                                                     kv_base, chunk_q, kv_total),
        }
        lim = [min(kv_total, kv_base + (i // chunk_q + 1) * chunk_q) if chunk_q else kv_total for i in range(Lq)]
        flops = 4.0 * br * H * sum(lim) * d
        for kind, op in ops.items():
            for _ in range(3):
                op()
            a, b = ev(), ev()
            torch.cuda.synchronize()
            a.record()
            for _ in range(20):
                op()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / 20 * 1e3
            out["%s_%s_us" % (name, kind)] = round(us, 2)
            out["%s_%s_tflops" % (name, kind)] = round(flops / (us * 1e-6) / 1e12, 1)
    print(json.dumps({"metric": "attention kernel time at the 40-layer step's shapes", "unit": "us", "n_gpus": 1,
                      "dtype": "bf16 and mxfp8", "data": "synthetic N(0,1)",
                      "config": {"workload": "2 x 40 heads, 464 queries; self 1392 keys chunk-causal, cross 769 keys"},
                      **out}))


def extra_workload(args, dev):
    """The other measured configurations (one JSON line each): one full-width block, four chunks of 16
    Euler steps, and the three-view long-context step; the default run measures the 40-layer CFG-2 step."""
    import numpy as np
    import torch

    import synth
    import world_action_video_amd as wam
    from synth.workloads import WORKLOADS, draw_named
    from world_action_video_amd.device import DeviceCache, DeviceCtx, DeviceModel, to_device, workspace

    w = WORKLOADS[args.workload]
    Lq, Lv, La = w.chunk_tokens, w.video_tokens, w.action_tokens

    def log(msg):
        print("[bench] %s" % msg, file=sys.stderr, flush=True)

    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)  # noqa: E731
    log("uploading %s weights" % w.name)
    model = DeviceModel(w, "bf16", dev, packed=not args.unpacked)
    ctx = DeviceCtx(w, "bf16", dev)
    ws = workspace(model.cfg, 1, dev)
    img = draw_named(w, -1, "img") if w.ctx_img_len else None
    wam.wam_ctx_build(model.cfg, model.weights, to_device(draw_named(w, -1, "txt"), "bf16", dev),
                      to_device(img, "bf16", dev) if img is not None else None, ctx.c, ws)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    base = {"n_gpus": 1, "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) weights, N(0,1) latents/features)",
            "config": {"workload": w.name + ("+unpacked-weights" if args.unpacked else ""), "layers": w.layers,
                       "dim": w.dim, "branches": w.branches, "chunk_tokens": Lq}}

    if args.workload == 2:
        # one block on the residual stream, CFG batch 2 and the B = 1 per-GPU share of a branch split
        res = {}
        for br in (2, 1):
            cfg = wam.wam_config.from_buffer_copy(model.cfg)
            cfg.branches = br
            cache = DeviceCache(w, 2 * Lq, "bf16", dev, branches=br)
            cx = DeviceCtx(w, "bf16", dev, branches=br)
            wsb = workspace(cfg, 1, dev)
            wam.wam_ctx_build(cfg, model.weights, to_device(draw_named(w, -1, "txt")[:br], "bf16", dev),
                              to_device(img, "bf16", dev), cx.c, wsb)
            wam.wam_kv_append(cfg, model.weights, cache.c, cx.c, f32(draw_named(w, -1, "x1_video_0")),
                              f32(draw_named(w, -1, "x1_action_0")), 0, wsb)
            h = torch.randn((br, Lq, w.dim), device=dev)
            e = torch.empty((2, w.dim), device=dev)
            e6 = torch.empty((2, 6, w.dim), device=dev)
            wam.wam_time_embed(cfg, model.weights, [0.4, 0.4], e, e6, wsb)
            blk = model.blocks[0]
            run = lambda: wam.wam_dit_block_fwd(cfg, blk, 0, cache.c, cx.c, h, e6, 1, w.frames_per_chunk, wsb)  # noqa
            for _ in range(args.warmup):
                run()
            a, b = ev(), ev()
            torch.cuda.synchronize()
            a.record()
            for _ in range(args.steps):
                run()
            b.record()
            torch.cuda.synchronize()
            res["br%d" % br] = round(a.elapsed_time(b) / args.steps, 3)
        out = dict(base, metric="ms per DiT block", value=res["br2"], unit="ms", higher_is_better=False,
                   ms_per_block={"cfg_batch_2": res["br2"], "B_1": res["br1"]})
        if not args.no_cpu_baseline:
            log("timing the oracle on the host")
            out["cpu_baseline"] = cpu_baseline(w.with_(layers=1))
        print(json.dumps(out))
        return

    n_new = 4 if args.workload == 4 else 1
    cache = DeviceCache(w, (w.cache_chunks + n_new) * Lq, "bf16", dev)
    for c in range(w.cache_chunks):
        wam.wam_kv_append(model.cfg, model.weights, cache.c, ctx.c, f32(draw_named(w, -1, "x1_video_%d" % c, n_chunks=8)),
                          f32(draw_named(w, -1, "x1_action_%d" % c, n_chunks=8)), c * w.frames_per_chunk, ws)
    vv = torch.empty((w.branches, Lv, w.patch_dim), device=dev)
    va = torch.empty((w.branches, La, w.action_dim), device=dev)
    gv = torch.empty(Lv * w.patch_dim, device=dev)
    ga = torch.empty(La * w.action_dim, device=dev)
    cos = torch.empty(3, device=dev)
    grid = [k / 16 for k in range(17)]
    torch.cuda.synchronize()

    if args.workload == 4:
        # four chunks: 16 Euler steps from noise, then the chunk is committed with a fresh video
        # observation and its own denoised actions
        times, calls = [], []
        xv0 = f32(draw_named(w, -1, "eps_video_1", n_chunks=8))
        xa0 = f32(draw_named(w, -1, "eps_action_1", n_chunks=8))
        xv, xa = xv0.clone(), xa0.clone()
        wam.wam_denoise_chunk(model.cfg, model.weights, cache.c, ctx.c, xv, xa, grid, w.guidance, 2.0, vv, va, gv, ga,
                              cos, ws, start_frame=w.frames_per_chunk)   # warm-up, cache untouched
        for c in range(1, 5):
            xv = f32(draw_named(w, -1, "eps_video_%d" % c, n_chunks=8))
            xa = f32(draw_named(w, -1, "eps_action_%d" % c, n_chunks=8))
            obs = f32(draw_named(w, -1, "x1_video_%d" % c, n_chunks=8))
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            n, _ = wam.wam_denoise_chunk(model.cfg, model.weights, cache.c, ctx.c, xv, xa, grid, w.guidance, 2.0, vv, va,
                                         gv, ga, cos, ws, start_frame=c * w.frames_per_chunk)
            wam.wam_kv_append(model.cfg, model.weights, cache.c, ctx.c, obs, xa, c * w.frames_per_chunk, ws)
            b.record()
            torch.cuda.synchronize()
            times.append(round(a.elapsed_time(b), 2))
            calls.append(n)
        finite = bool(torch.isfinite(xv).all().item() and torch.isfinite(xa).all().item())
        out = dict(base, metric="ms per chunk (16 Euler steps + KV append)", value=round(sum(times) / 4, 2), unit="ms",
                   higher_is_better=False, per_chunk_ms=times, total_ms=round(sum(times), 1), dit_calls=calls,
                   cache_rows_final=cache.length, outputs_finite=finite)
        if not args.no_cpu_baseline:
            log("timing the oracle on the host")
            cb = cpu_baseline(w)
            cb["sample"] += ("; one chunk extrapolated as 17 steps at the first chunk's cache (16 DiT calls plus "
                             "the append's pass), not run")
            cb["value"] = round(cb["value"] * 17, 1)
            cb["unit"] = "ms per chunk (extrapolated)"
            out["cpu_baseline"] = cb
        print(json.dumps(out))
        return

    # three-view long context: one step with decoupled timesteps, then a 16-step loop with velocity reuse
    start = w.cache_chunks * w.frames_per_chunk
    xv = f32(draw_named(w, -1, "eps_video_%d" % w.cache_chunks, n_chunks=8))
    xa = f32(draw_named(w, -1, "eps_action_%d" % w.cache_chunks, n_chunks=8))
    u = synth.uniform01(2 * (args.steps + args.warmup), synth.tensor_key(w.id, -1, "timesteps"), stream=2)
    tv = 1.0 - np.sqrt(u[0::2])          # sigma = 1 - t_v ~ Beta(2, 1): inverse CDF of x^2
    ta = u[1::2]
    for i in range(args.warmup):
        wam.wam_dit_stack_fwd(model.cfg, model.weights, cache.c, ctx.c, 1, xv, xa, [tv[i]], [ta[i]], start, vv, va, ws)
    a, b = ev(), ev()
    torch.cuda.synchronize()
    a.record()
    for i in range(args.steps):
        j = args.warmup + i
        wam.wam_dit_stack_fwd(model.cfg, model.weights, cache.c, ctx.c, 1, xv, xa, [tv[j]], [ta[j]], start, vv, va, ws)
    b.record()
    torch.cuda.synchronize()
    step_ms = a.elapsed_time(b) / args.steps
    a, b = ev(), ev()
    a.record()
    n, flags = wam.wam_denoise_chunk(model.cfg, model.weights, cache.c, ctx.c, xv, xa, grid, w.guidance, 0.99, vv, va,
                                     gv, ga, cos, ws, start_frame=start)
    b.record()
    torch.cuda.synchronize()
    loop_ms = a.elapsed_time(b)
    finite = bool(torch.isfinite(xv).all().item() and torch.isfinite(xa).all().item())
    out = dict(base, metric="ms per DiT denoise step (40L, CFG b=2, 8064 cached tokens)", value=round(step_ms, 3),
               unit="ms", higher_is_better=False, loop_16_steps_ms=round(loop_ms, 1), dit_calls=n,
               reused_steps=[k for k, f in enumerate(flags) if f], cached_tokens=cache.length, outputs_finite=finite)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
