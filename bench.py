"""Benchmark of the block-sparse attention forward layer on one MI355X.

One step = the whole path over one layer's Q/K/V already resident in HBM:
block means of Q and K (one read each), reorder V into channel-major blocks in the
same launch (unless the first call's mask selected reading V in the original order),
build the mask, block-sparse attention reading Q and K in the original order and
writing O in the original order. `timed_steps_ms` lists each timed step's duration.

Prints ONE JSON line. `value` is the dense-equivalent throughput
4*B*H*N^2*d / (time per layer); `ms_per_step` is the time per layer. Steps are
launched eagerly; with --graph each step replays the whole path captured once in a
HIP graph, and `ms_per_layer_eager` then gives the eager time for comparison.
The `roofline` object is for the attention kernel (the dominant one): the
FLOPs of the kept 64x64 blocks per launch over its average launch time, timed
with HIP events on the stream the kernels run on. `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload and scales it to the layer.

Usage: python bench.py [--gpus 1] [--steps 10] [--warmup 20] [--workload 480p] [--secondary 720p] [--graph]
       python bench.py --report          (per-pass table over every workload, and the backward)
       python bench.py --backward --workload 720p   (abla_sparse_attn_bwd timing, one JSON line)
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
FP32_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (a few ms of load is not enough for the clocks to settle)")
    ap.add_argument("--workload", default="480p")
    ap.add_argument("--secondary", default="720p", help="second workload reported alongside ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample (0: skip)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per attention launch (from rocprofv3 counters)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step captured in a HIP graph instead of launching it eagerly")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (abla_sparse_attn_bwd) on --workload instead; one JSON line")
    ap.add_argument("--report", action="store_true",
                    help="instead of the JSON line, print a markdown report over every workload (and the "
                         "dynamic-threshold sweep) with per-pass times, fractions and per-head keep")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for the FETCH/WRITE_SIZE counters)")
    return ap.parse_args()


def copy_calibration(mib, reps=5):
    """A plain copy of a known size: under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE per dispatch
    give the factor that turns the counters into bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src), reps, torch.cuda.current_stream())
    print(json.dumps({"copy_bytes": n * 4, "reps": reps, "ms": round(ms, 4),
                      "GB/s (read+write)": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}), flush=True)


def timed(fn, reps, stream):
    """Average milliseconds of fn() over reps launches, HIP events on `stream`."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def per_launch(fn, reps, stream, flush=None):
    """Milliseconds of each of reps launches of fn(), HIP events on `stream` around each one;
    flush(), when given, runs before each launch outside its events."""
    import torch
    pairs = []
    torch.cuda.synchronize()
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in pairs)


def _probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_21_amd", "libabla_probe.so"))
    lib.abla_probe_mfma.restype = ctypes.c_int32
    lib.abla_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.abla_probe_mfma_flops.restype = ctypes.c_double
    lib.abla_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.abla_probe_stream.restype = ctypes.c_int32
    lib.abla_probe_stream.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
    return lib


def hbm_stream_peak(copy, mib=2048, warm=3, reps=10):
    """Sustained HBM rate on this board (GB/s): libabla_probe's stream of 16-byte loads over `mib`
    MiB (8x the last-level cache), 32 KiB per workgroup, read-only or a copy (read + write bytes)."""
    import ctypes
    import torch
    lib = _probe_lib()
    nbytes = mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty(nbytes // 4 if copy else 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        rc = lib.abla_probe_stream(int(copy), ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                   nbytes, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"abla_probe_stream failed ({rc})")

    for _ in range(warm):
        launch()
    ms = timed(launch, reps, stream)
    return nbytes * (2 if copy else 1) / (ms * 1e-3) / 1e9


def graph_ms(fn, launches=10, reps=5):
    """Milliseconds per call of fn() with launch gaps removed: `launches` calls captured in one
    HIP graph, replayed `reps` times (fn must be capturable: no allocation, no memset)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            fn()
    g.replay()
    return timed(g.replay, reps, torch.cuda.current_stream()) / launches


def mfma_loop_peak(kind=0, grid=2048, iters=20000, warm=12, reps=8):
    """Sustained matrix-core rate on this board (TFLOP/s): libabla_probe's loop of independent
    MFMAs with no memory traffic (kind 0: bf16 32x32x16, kind 1: float32 32x32x2), eight
    workgroups per CU, timed with HIP events after enough launches for the clocks to settle."""
    import ctypes
    import torch
    lib = _probe_lib()
    sink = torch.zeros(grid, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        rc = lib.abla_probe_mfma(kind, grid, iters, ctypes.c_void_p(sink.data_ptr()),
                                 ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"abla_probe_mfma failed ({rc})")

    for _ in range(warm):
        launch()
    ms = timed(launch, reps, stream)
    return lib.abla_probe_mfma_flops(kind, grid, iters) / (ms * 1e-3) / 1e12


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


# Bytes written between launches of the cold-cache timing: twice the 256 MB last-level cache.
EVICT_BYTES = 512 << 20


def measure(name, steps, warmup, use_graph=False):
    import torch
    import block_sparse_attention_21_amd as A
    from gen import WORKLOADS, make_qkv

    w = WORKLOADS[name] if isinstance(name, str) else name
    geom = A.Geometry(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    prm = A.MaskParams(mode=w.mode, thr=w.thr, tau=w.tau, sta=tuple(w.sta), gamma=w.gamma, lam=w.lam)
    q, k, v = make_qkv(w, device="cuda")
    run = A.NablaAttention(geom, prm, dtype=q.dtype)
    stream = torch.cuda.current_stream()
    # One step = the whole path on resident inputs, launched eagerly, or with --graph replayed
    # from a HIP graph (same kernels, same arguments; measured no faster on this path).
    graph = run.capture(q, k, v) if use_graph else None
    step = graph.replay if graph is not None else (lambda: run(q, k, v))
    for _ in range(warmup):
        step()
    if run._decide_v:  # no warm-up step made the V-path choice: make it outside the timed region
        run(q, k, v)
    torch.cuda.synchronize()

    # The timed region: exactly `steps` whole-path steps. Eagerly launched, each step's attention
    # call (the visiting-order kernel and the attention kernel) sits between two HIP events on
    # the stream, which gives the attention's duration inside the layer from the same steps.
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    done = []

    def step_marked():
        starts[len(done)].record(stream)
        run.reorder_pool(q, k, v)
        run.mask()
        a, b = marks[len(done)]
        a.record(stream)
        run.attend()
        b.record(stream)
        done.append(1)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = timed(step if graph is not None else step_marked, steps, stream)
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms_attn_layer = sum(a.elapsed_time(b) for a, b in marks) / steps if graph is None else None
    # Each timed step from its start to the next step's start (the last one to its attention's end).
    step_ms = ([starts[i].elapsed_time(starts[i + 1]) for i in range(steps - 1)]
               + [starts[-1].elapsed_time(marks[-1][1])]) if graph is None else None
    ms_eager = timed(lambda: run(q, k, v), steps, stream) if graph is not None else ms_step

    # Per-stage averages (same inputs, state left by the path).
    ms_reorder = timed(lambda: run.reorder_pool(q, k, v), steps, stream)
    ms_reorder_graph = graph_ms(lambda: run.reorder_pool(q, k, v))
    ms_mask = timed(run.mask, steps, stream)
    ms_mask_graph = graph_ms(run.mask)
    ms_attn_stage = timed(run.attend, steps, stream)  # back to back, no other stage between
    ms_attn = ms_attn_layer if ms_attn_layer is not None else ms_attn_stage

    # Then the spread of single steps, and single steps each started after writing EVICT_BYTES
    # of scratch (so no input is left in the last-level cache).
    warm = per_launch(step, steps, stream)
    scratch = torch.empty(EVICT_BYTES // 4, dtype=torch.float32, device="cuda")
    cold = per_launch(step, steps, stream, flush=lambda: scratch.fill_(1.0))
    del scratch

    kept = int(run.counts.sum().item())
    total = w.B * w.H * w.nb * w.nb
    dense = A.dense_flops(geom)
    kept_fl = A.kept_flops(geom, kept)
    elem = 2 if w.dtype == "bf16" else 4
    tensor_bytes = w.B * w.H * w.N * w.d * elem
    pooled_bytes = w.B * w.H * w.nb * w.d * 8
    # Q and K are read once for pooling (the attention reads them in the original order); V is
    # read and written channel-major unless the attention reads it in the original order; plus
    # the pooled means.
    reorder_bytes = (2 if run.fuse_v else 4) * tensor_bytes + 2 * pooled_bytes
    return dict(
        w=w, geom=geom, kept=kept, keep_fraction=kept / total, ms_step=ms_step, wall_ms_step=wall, ms_eager=ms_eager,
        graph=graph is not None, warm=warm, cold=cold,
        ms_reorder=ms_reorder, ms_mask=ms_mask, ms_mask_graph=ms_mask_graph, ms_attn=ms_attn,
        ms_attn_stage=ms_attn_stage,
        attn_in_layer=ms_attn_layer is not None, dense_flops=dense, kept_flops=kept_fl,
        reorder_gbs=reorder_bytes / (ms_reorder * 1e-3) / 1e9, tensor_bytes=tensor_bytes, reorder_bytes=reorder_bytes,
        ms_reorder_graph=ms_reorder_graph, reorder_gbs_graph=reorder_bytes / (ms_reorder_graph * 1e-3) / 1e9,
        counts=run.counts, run=run, q=q, k=k, v=v, v_original=run.fuse_v, step_ms=step_ms,
    )


def measure_backward(w, steps, warmup):
    """Time abla_sparse_attn_bwd (all its passes) after one forward, on the same workload, with
    a seeded incoming gradient. Algorithmic FLOPs: 10*64*64*d per kept block pair (S, dP, dV,
    dK, dQ); the kernels issue 14*64*64*d (S and dP are formed once for dQ and once for dK/dV)."""
    import torch
    import block_sparse_attention_21_amd as A
    from gen import make_dout, make_qkv

    geom = A.Geometry(w.B, w.H, w.T, w.Hs, w.Ws, w.d, w.P)
    prm = A.MaskParams(mode=w.mode, thr=w.thr, tau=w.tau, sta=tuple(w.sta), gamma=w.gamma, lam=w.lam)
    q, k, v = make_qkv(w, device="cuda")
    dout = make_dout(w.B, w.H, geom.N, w.d, seed=7, device="cuda")
    run = A.NablaAttention(geom, prm, dtype=q.dtype, want_lse=True)
    run(q, k, v)
    ws = torch.empty(A.sparse_attn_bwd_workspace_bytes(geom), dtype=torch.uint8, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def bwd():
        A.sparse_attn_bwd(q, k, v, run.out, dout, run.lse, run.words, run.counts, run.lists, geom,
                          dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(warmup):
        bwd()
    ms = timed(bwd, steps, torch.cuda.current_stream())
    kept = int(run.counts.sum().item())
    return dict(kept=kept, ms=ms, alg_flops=10.0 * 64 * 64 * w.d * kept, mfma_flops=14.0 * 64 * 64 * w.d * kept)


def cpu_baseline(r, budget_s):
    """Time the CPU oracle on a bounded sample (one head: pool + mask in full, attention on sampled
    query blocks until the budget is spent) and scale it to the whole layer."""
    import numpy as np
    from oracle import nabla_ref as R

    w = r["w"]
    cores = len(os.sched_getaffinity(0))
    blas = {}
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threadpool_limits(cores)  # every BLAS pool at the cores this process may use
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if pools:
            blas = {"blas": f"{pools[0].get('internal_api')} {pools[0].get('version')}",
                    "blas_threads": int(pools[0].get("num_threads", cores))}
    except Exception:
        pass
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    g1 = R.Geom(1, 1, w.T, w.Hs, w.Ws, w.d, w.P)
    prm = R.MaskParams(mode=w.mode, thr=w.thr, tau=w.tau, sta=tuple(w.sta), gamma=w.gamma, lam=w.lam)
    q, k, v = (x[0, 0].float().cpu().numpy().astype(np.float64) for x in (r["q"], r["k"], r["v"]))
    t0 = time.perf_counter()
    Qr, Kr, Vr = R.reorder(q, g1), R.reorder(k, g1), R.reorder(v, g1)
    qbar, kbar = R.block_means(Qr, g1), R.block_means(Kr, g1)
    mres = R.build_block_mask(qbar[None, None], kbar[None, None], g1, prm)
    t_mask = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    blocks = rng.permutation(g1.nb)
    done = 0
    t1 = time.perf_counter()
    scale = 1.0 / math.sqrt(w.d)
    while done < g1.nb and (time.perf_counter() - t1) < budget_s:
        b = int(blocks[done])
        R.masked_attention_head(Qr, Kr, Vr, mres.mask[0, 0], g1, scale, rows=np.arange(b * 64, (b + 1) * 64))
        done += 1
    t_attn = time.perf_counter() - t1
    head_s = t_mask + t_attn * g1.nb / max(done, 1)
    layer_s = head_s * w.B * w.H
    return {
        "value": r["dense_flops"] / layer_s / 1e12, "unit": "TFLOP/s (dense-equivalent)",
        "cores": int(blas.get("blas_threads", cores)), "affinity_cores": cores, "cpu_model": cpu_model,
        "blas": blas.get("blas", "unknown"), "kind": "oracle", "ms_per_layer_est": layer_s * 1e3,
        "sample": f"1 of {w.B * w.H} heads: reorder+pool+mask in full ({t_mask:.2f} s) and masked attention on "
                  f"{done} of {g1.nb} query blocks ({t_attn:.2f} s), scaled by blocks and heads; float64 numpy",
    }


def report(args):
    """Markdown report over every workload: per-pass times, dense-equivalent and actual TFLOP/s,
    MFMA fraction (against the 2.5 PFLOP/s datasheet peak and against a large bf16 library GEMM
    timed on the same board), HBM fractions of the reorder and mask passes, keep per head."""
    import torch
    from gen import WORKLOADS

    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(20):
        torch.matmul(a, b)
    gemm = 2.0 * n ** 3 / (timed(lambda: torch.matmul(a, b), 20, torch.cuda.current_stream()) * 1e-3) / 1e12
    del a, b
    cases = [WORKLOADS["tiny"], WORKLOADS["480p"], WORKLOADS["720p"], WORKLOADS["480p-dyn"],
             WORKLOADS["480p-dyn"].with_(tau=2.0), WORKLOADS["480p-dyn"].with_(tau=8.0), WORKLOADS["480p-static"],
             WORKLOADS["long"]]
    loop_bf16, loop_f32 = mfma_loop_peak(0), mfma_loop_peak(1)
    hbm_read, hbm_copy = hbm_stream_peak(False), hbm_stream_peak(True)
    print(f"bf16 GEMM reference (torch.matmul {n}^3): {gemm:,.0f} TFLOP/s; matrix-core loops on this board "
          f"(libabla_probe, no memory traffic): bf16 {loop_bf16:,.0f} TFLOP/s, float32 {loop_f32:,.1f} TFLOP/s "
          f"(datasheet {MFMA_BF16_PEAK_TFLOPS:,.0f} / {FP32_PEAK_TFLOPS}); HBM streams (libabla_probe, 2 GiB): "
          f"read {hbm_read:,.0f} GB/s, copy {hbm_copy:,.0f} GB/s (datasheet {HBM_PEAK_GBS:,.0f})\n")
    fwd_attn_ms = {}
    print("| workload | mask | keep | first step ms (TB/s); kernel-only from a graph | mask ms (GB/s); from a graph | "
          "attention ms: in the layer / back to back | layer ms | "
          "single layers: median / min / cold median ms | "
          "dense-eq TFLOP/s (layer / attn) | actual TFLOP/s | of datasheet peak | of MFMA loop | of GEMM ref | "
          "keep per head |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for w in cases:
        r = measure(w, args.steps, args.warmup)
        g = r["geom"]
        counts = r["counts"].double()
        per_head = (counts.sum(dim=-1) / (g.nb * g.nb)).flatten().cpu().tolist()
        e = 2 if w.dtype == "bf16" else 4
        pooled = g.B * g.H * g.nb * g.d * 8
        out_bytes = g.B * g.H * g.nb * (g.words + 1) * 4 + r["kept"] * 4  # words, counts, lists
        # Scored modes also read the pooled vectors and write + read the float64 score matrix.
        mask_bytes = out_bytes + (0 if w.mode == "static" else 2 * pooled + 2 * g.B * g.H * g.nb * g.nb * 8)
        attn_tf = r["kept_flops"] / (r["ms_attn"] * 1e-3) / 1e12
        peak, loop = (MFMA_BF16_PEAK_TFLOPS, loop_bf16) if w.dtype == "bf16" else (FP32_PEAK_TFLOPS, loop_f32)
        mode = {"cdf": f"cdf {w.thr}", "dyn": f"dyn tau={w.tau}",
                "static": f"static gamma={w.gamma} lambda={w.lam}"}[w.mode]
        heads = ", ".join(f"{x:.3f}" for x in per_head[:12]) + (" ..." if len(per_head) > 12 else "")
        vpath = "V original order" if r["v_original"] else "V pass"
        print(f"| {w.name} ({w.dtype}, {w.N} tok; {vpath}) | {mode} | {r['keep_fraction']:.4f} | "
              f"{r['ms_reorder']:.4f} ({r['reorder_gbs'] / 1e3:.2f}); {r['ms_reorder_graph']:.4f} "
              f"({r['reorder_gbs_graph'] / 1e3:.2f}) | {r['ms_mask']:.4f} "
              f"({mask_bytes / (r['ms_mask'] * 1e-3) / 1e9:,.0f}); {r['ms_mask_graph']:.4f} | "
              f"{r['ms_attn']:.4f} / {r['ms_attn_stage']:.4f} | "
              f"{r['ms_step']:.4f} | "
              f"{median(r['warm']):.4f} / {r['warm'][0]:.4f} / {median(r['cold']):.4f} | "
              f"{r['dense_flops'] / (r['ms_step'] * 1e-3) / 1e12:,.1f} / "
              f"{r['dense_flops'] / (r['ms_attn'] * 1e-3) / 1e12:,.1f} | {attn_tf:,.1f} | "
              f"{attn_tf / peak:.3f} | {attn_tf / loop:.3f} | {attn_tf / gemm:.3f} | {heads} |", flush=True)
        fwd_attn_ms[w.name + (f"-tau{w.tau}" if w.mode == "dyn" else "")] = r["ms_attn"]
        del r
    print("\nBackward (abla_sparse_attn_bwd, every pass: D and L2 rows, column lists, visiting order, dQ, dK+dV), "
          "bf16 workloads:\n")
    print("| workload | keep | backward ms | algorithmic TFLOP/s (10*64^2*d per kept pair) | of 2.5 PF | "
          "issued MFMA TFLOP/s (14*64^2*d) | backward / forward attention |")
    print("|---|---|---|---|---|---|---|")
    for w in cases:
        if w.dtype != "bf16":
            continue
        b = measure_backward(w, args.steps, args.warmup)
        key = w.name + (f"-tau{w.tau}" if w.mode == "dyn" else "")
        alg = b["alg_flops"] / (b["ms"] * 1e-3) / 1e12
        print(f"| {key} | {b['kept'] / (w.B * w.H * w.nb * w.nb):.4f} | {b['ms']:.3f} | {alg:,.1f} | "
              f"{alg / MFMA_BF16_PEAK_TFLOPS:.3f} | {b['mfma_flops'] / (b['ms'] * 1e-3) / 1e12:,.1f} | "
              f"{b['ms'] / fwd_attn_ms[key]:.2f} |", flush=True)


def traffic_for(path, name):
    try:
        with open(path) as f:
            return json.load(f).get(name)
    except (OSError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus above 1 is not supported"}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no HIP device"}))
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.report:
        report(args)
        return
    if args.backward:
        from gen import WORKLOADS
        w = WORKLOADS[args.workload]
        b = measure_backward(w, args.steps, args.warmup)
        alg = b["alg_flops"] / (b["ms"] * 1e-3) / 1e12
        print(json.dumps({
            "what": "block-sparse attention backward (abla_sparse_attn_bwd, every pass)", "workload": w.name,
            "steps": args.steps, "warmup": args.warmup, "ms": round(b["ms"], 4), "kept_pairs": b["kept"],
            "algorithmic_tflops": round(alg, 2), "frac_of_2.5PF": round(alg / MFMA_BF16_PEAK_TFLOPS, 4),
            "issued_mfma_tflops": round(b["mfma_flops"] / (b["ms"] * 1e-3) / 1e12, 2),
        }), flush=True)
        return
    r = measure(args.workload, args.steps, args.warmup, use_graph=args.graph)
    w, geom = r["w"], r["geom"]
    f32 = w.dtype == "f32"
    loop_peak = mfma_loop_peak(1 if f32 else 0)
    peak = FP32_PEAK_TFLOPS if f32 else MFMA_BF16_PEAK_TFLOPS
    hbm_read, hbm_copy = hbm_stream_peak(False), hbm_stream_peak(True)
    value = r["dense_flops"] / (r["ms_step"] * 1e-3) / 1e12
    attn_tflops = r["kept_flops"] / (r["ms_attn"] * 1e-3) / 1e12
    traffic = traffic_for(args.traffic, w.name)
    out = {
        "metric": f"effective TFLOP/s (dense-equivalent 4*B*H*N^2*d per layer), block-sparse attention forward "
                  f"layer at {w.N} tokens",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded smooth spatio-temporal Q/K field with long-range block copies, V~N(0,1))",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "T": w.T, "Hs": w.Hs, "Ws": w.Ws, "d": w.d, "tokens": w.N,
            "blocks": w.nb, "mask": w.mode, "thr": w.thr if w.mode == "cdf" else None,
            "tau": w.tau if w.mode == "dyn" else None, "sta": list(w.sta), "parallelism": "none (1 GPU)",
            "launch": "hip graph replay of the whole step" if r["graph"] else "eager",
            "v_read": "original order (no V pass)" if r["v_original"] else "channel-major blocks (V pass)",
        },
        "ms_per_layer": round(r["ms_step"], 4),
        "ms_per_layer_eager": round(r["ms_eager"], 4),
        "timed_steps_ms": [round(x, 4) for x in r["step_ms"]] if r["step_ms"] is not None else None,
        "single_steps": {"reps": len(r["warm"]), "ms_median": round(median(r["warm"]), 4),
                         "ms_min": round(r["warm"][0], 4)},
        "cold_cache": {"reps": len(r["cold"]), "evict_bytes": EVICT_BYTES, "ms_median": round(median(r["cold"]), 4),
                       "ms_min": round(r["cold"][0], 4)},
        "ms_per_stage": {"reorder_pool_qkv": round(r["ms_reorder"], 4), "mask": round(r["ms_mask"], 4),
                         "mask_kernel_graph": round(r["ms_mask_graph"], 4),
                         "attention": round(r["ms_attn_stage"], 4)},
        "ms_attention_in_layer": round(r["ms_attn"], 4) if r["attn_in_layer"] else None,
        "keep_fraction": round(r["keep_fraction"], 5),
        "attention_actual_tflops": round(attn_tflops, 2),
        "reorder_pool_gbs": round(r["reorder_gbs"], 1),
        "first_step": {
            "kernel": "k_pool_qk_reorder_v (pool Q and K" + (")" if r["v_original"] else ", reorder V)"),
            "bound": "hbm", "bytes": int(r["reorder_bytes"]),
            "gbs_stage": round(r["reorder_gbs"], 1),
            "gbs_kernel_graph": round(r["reorder_gbs_graph"], 1),
            "ms_kernel_graph": round(r["ms_reorder_graph"], 4),
            "peak": HBM_PEAK_GBS, "frac_kernel": round(r["reorder_gbs_graph"] / HBM_PEAK_GBS, 4),
            "hbm_read_probe_gbs": round(hbm_read, 1), "hbm_copy_probe_gbs": round(hbm_copy, 1),
        },
        "roofline": {
            "kernel": ("k_attn_f32" if f32 else "k_attn_bf16") + " (block-sparse attention forward)",
            "bound": "mfma",
            "ms_per_launch": round(r["ms_attn"], 4),
            "timing": ("HIP events around the attention entry point (visiting-order kernel + attention kernel) "
                       "inside each timed step" if r["attn_in_layer"] else
                       "HIP events around back-to-back attention entry-point calls (graph mode)"),
            "achieved": round(attn_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": traffic,
            "mfma_loop_peak": round(loop_peak, 1),
            "frac_of_mfma_loop": round(attn_tflops / loop_peak, 4),
        },
    }
    if args.secondary:
        s = measure(args.secondary, args.steps, args.warmup, use_graph=args.graph)
        out["secondary"] = {
            "workload": s["w"].name, "tokens": s["w"].N, "ms_per_layer": round(s["ms_step"], 4),
            "effective_tflops": round(s["dense_flops"] / (s["ms_step"] * 1e-3) / 1e12, 3),
            "attention_actual_tflops": round(s["kept_flops"] / (s["ms_attn"] * 1e-3) / 1e12, 2),
            "mfma_frac": round(s["kept_flops"] / (s["ms_attn"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "frac_of_mfma_loop": (round(s["kept_flops"] / (s["ms_attn"] * 1e-3) / 1e12 / loop_peak, 4)
                                  if s["w"].dtype == w.dtype else None),
            "keep_fraction": round(s["keep_fraction"], 5),
            "ms_per_stage": {"reorder_pool_qkv": round(s["ms_reorder"], 4), "mask": round(s["ms_mask"], 4),
                             "mask_kernel_graph": round(s["ms_mask_graph"], 4),
                             "attention": round(s["ms_attn_stage"], 4)},
            "ms_attention_in_layer": round(s["ms_attn"], 4) if s["attn_in_layer"] else None,
            "reorder_pool_gbs": round(s["reorder_gbs"], 1),
            "reorder_pool_gbs_kernel_graph": round(s["reorder_gbs_graph"], 1),
            "single_steps_ms_median": round(median(s["warm"]), 4),
            "cold_cache_ms_median": round(median(s["cold"]), 4),
        }
        del s
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(r, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
