"""Benchmark of the single-GPU MoE layer forward (HIP path) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--configs A,B,..|none]
                    [--no-cpu-baseline] [--graph-steps G] [--backward-steps B]

A step is one full moe_forward (router, capacity scan, dispatch, expert GEMM 1 + act, expert
GEMM 2, combine + aux) over one batch of seeded synthetic tokens already resident in HBM, with
4 rotating copies of x and y (each step also streams every expert's weights, so the 256 MB
MALL does not hold the next step's inputs).  W untimed steps, then K timed steps bracketed by
torch.cuda.synchronize().  The library records HIP events at the stage boundaries on the
launch stream; a step's time is the event time from its first launch to its last, and the
reported layer time is the median over the K steps (the wall time of the K steps between the
two synchronisations is reported beside it).

The headline (value, roofline, cpu_baseline) is the large-expert layer, the largest
configuration; the other reference layers are measured in the same run, each in its own
object under "configs" with the same fields.

roofline: the dominant kernel, the expert GEMM (two launches per step, GEMM 1 with the
activation and GEMM 2).  Algorithmic flops per launch: 2 R M H for the routed rows (R = kept
rows) + 2 N Es H M for the shared experts, doubled in the gated experts' GEMM 1; algorithmic
bytes: the activations read and written once plus the weights of every expert that received
rows.  Both over the average launch time (HIP events).  The bound is the one each layer's
shapes give: MFMA for the large-expert, GShard-style and shared+routed layers, HBM for the
Switch-style layer, whose 1.2 GB of weights feed at most 256 flop per byte.
cpu_baseline: the CPU oracle, as it stands, timed on a bounded sample of the same workload.
graph: the same forward step replayed from HIP graphs; backward: moe_backward timed on the same
inputs (routing and expert activations recomputed, all gradients).
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mixture_experts_layer_group_amd import binding, configs, synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (MFMA and vector)
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_gemm_traffic.json")
HEADLINE = configs.BENCH_WORKLOAD
OTHER_CONFIGS = ("tiny_fp32", "gshard_bf16", "switch_bf16", "shared_routed_bf16")
# Roofline bound of the expert GEMM per layer: the Switch-style layer streams 1.2 GB of expert
# weights for at most 0.31 TFLOP (<= 256 flop/B, under the 312 flop/B ridge); the others are
# contractions that the MFMA peak bounds.
FFN_BOUND = {"switch_bf16": "hbm"}


class HipEvents:
    """hipEvent_t handles through the HIP runtime (timing events on the launch stream)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h)
        return out

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)


def kernel_hash():
    h = hashlib.sha256()
    for f in ("moe_expert_ffn.hip", "moe_device.h", "moe_internal.h", "moe_tile_map.h"):
        with open(os.path.join(ROOT, "mixture_experts_layer_group_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per expert-GEMM launch of a workload from the committed rocprofv3 counter
    summary, or None when the counters were taken on another kernel version or not on this
    workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash():
        return None
    w = t.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def ffn_flops_per_token(cfg):
    """Oracle FFN flops of one token with every slot kept (routed + shared experts)."""
    M, H, k, Es = cfg["d_model"], cfg["d_ff"], cfg["top_k"], cfg["n_shared"]
    gl = 2 if cfg["act"] == configs.ACT_SWIGLU else 1
    return (k + Es) * (gl + 1) * 2.0 * M * H


def cpu_baseline(cfg, inp, budget_tokens, min_seconds=10.0, max_passes=20):
    """Time the CPU oracle as it stands: router logits + routing + positions + aux over all N
    tokens, expert FFN + combine over a seeded sample of budget_tokens tokens, repeated until
    ~min_seconds of CPU work has been timed."""
    from oracle import moe_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas_threads = 1
    N = cfg["n_tokens"]
    ns = max(1, min(N, budget_tokens))
    toks = np.sort(np.random.default_rng(1).choice(N, size=ns, replace=False))
    t_route = t_ffn = 0.0
    passes = 0
    while passes < max_passes and (passes == 0 or t_route + t_ffn < min_seconds):
        t0 = time.perf_counter()
        logits = mo.router_logits(inp.x, inp.Wg, inp.bg)
        r = mo.route(cfg, logits.astype(np.float32), inp.u)
        t1 = time.perf_counter()
        mo.layer_outputs(cfg, inp.x, inp.W1, inp.W2, r, tokens=toks)
        t2 = time.perf_counter()
        t_route += t1 - t0
        t_ffn += t2 - t1
        passes += 1
    per_token = (t_route / N + t_ffn / ns) / passes
    return {"value": round(1.0 / per_token, 1), "unit": "tokens/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": (f"float64 NumPy oracle, {passes} passes: router logits + routing + "
                       f"positions + aux over all {N} tokens ({t_route / passes:.2f} s/pass), "
                       f"expert FFN + combine over a seeded sample of {ns} tokens "
                       f"({t_ffn / passes:.2f} s/pass); tokens/s = 1 / (route s/token + FFN "
                       f"s/token); host: {cpu_model()}, os.cpu_count()={os.cpu_count()}, BLAS "
                       f"threads={blas_threads}")}


def backward_timing(cfg, x, Wg, W1, W2, bg, u, R, steps):
    """Time moe_backward (routing and expert activations recomputed, all gradients) on the
    same inputs with a seeded dy; both aux-loss coefficients nonzero.  Algorithmic expert flops
    of the backward proper: dgrad + wgrad = 2x the forward FFN's; the recompute adds GEMM 1
    only (the combine weights' gradient comes out of the dgrad GEMM, not from recomputed
    expert outputs)."""
    import torch
    dy32, dybits = synth.upstream_grad(cfg)
    dy = (torch.from_numpy(dybits.view(np.int16)).cuda().view(torch.bfloat16)
          if dybits is not None else torch.from_numpy(dy32).cuda())
    ws = torch.empty(binding.moe_backward_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    meta = binding.alloc_meta(cfg)
    coefs = dict(coef_aux=0.01, coef_z=0.001, coef_dev=0.0)
    out, _ = binding.backward(cfg, x, Wg, W1, W2, dy, bg=bg, u=u, workspace=ws, meta=meta,
                              **coefs)
    torch.cuda.synchronize()
    ms = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        binding.moe_backward(cfg, x, Wg, bg, W1, W2, u, dy, coefs["coef_aux"], coefs["coef_z"],
                             coefs["coef_dev"], out["dx"], out["dWg"], out["dbg"], out["dW1"],
                             out["dW2"], meta, ws)
        e1.record()
        ms.append((e0, e1))
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in ms]))
    # the training pair: moe_forward_train keeps h (and z) in the workspace, then
    # moe_backward_saved skips GEMM 1; each call timed on its own
    y = torch.empty_like(x)
    aux = torch.empty((4,), dtype=torch.float32, device="cuda")
    tf, tb = [], []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        binding.moe_forward_train(cfg, x, Wg, bg, W1, W2, u, y, aux, meta, ws)
        e[1].record()
        binding.moe_backward_saved(cfg, x, Wg, bg, W1, W2, u, dy, coefs["coef_aux"],
                                   coefs["coef_z"], coefs["coef_dev"], out["dx"], out["dWg"],
                                   out["dbg"], out["dW1"], out["dW2"], meta, ws)
        e[2].record()
        tf.append((e[0], e[1]))
        tb.append((e[1], e[2]))
    torch.cuda.synchronize()
    t_tf = float(np.median([a.elapsed_time(b) for a, b in tf]))
    t_bs = float(np.median([a.elapsed_time(b) for a, b in tb]))
    N, M, H, Es = cfg["n_tokens"], cfg["d_model"], cfg["d_ff"], cfg["n_shared"]
    gl = 2 if cfg["act"] == configs.ACT_SWIGLU else 1
    fwd_ffn = (gl + 1) * 2.0 * M * H * (R + N * Es)
    recompute = gl * 2.0 * M * H * (R + N * Es)
    del out, ws, dy, y, aux
    return {"ms": round(t, 4), "tokens_per_s": round(N / (t * 1e-3), 1), "steps": steps,
            "timing": "median of per-call HIP events",
            "ffn_flops_backward": 2 * fwd_ffn, "ffn_flops_recompute": recompute,
            "tflops_backward_alg": round(2 * fwd_ffn / (t * 1e-3) / 1e12, 2),
            "tflops_incl_recompute": round((2 * fwd_ffn + recompute) / (t * 1e-3) / 1e12, 2),
            "saved": {"backward_ms": round(t_bs, 4), "forward_train_ms": round(t_tf, 4),
                      "tflops_backward_alg": round(2 * fwd_ffn / (t_bs * 1e-3) / 1e12, 2),
                      "note": "moe_forward_train then moe_backward_saved (expert activations "
                              "kept by the forward, GEMM 1 not recomputed)"}}


def graph_timing(cfg, xs, ys, Wg, bg, W1, W2, u, aux, meta, ws, steps):
    """The same forward step replayed from HIP graphs (one captured moe_forward per rotating
    x/y copy), which removes the host launch work between the five kernels."""
    import torch
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        binding.moe_forward(cfg, xs[0], Wg, bg, W1, W2, u, ys[0], aux, meta, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for c in range(len(xs)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            binding.moe_forward(cfg, xs[c], Wg, bg, W1, W2, u, ys[c], aux, meta, ws)
        graphs.append(g)
    for i in range(2 * len(graphs)):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del graphs
    return {"ms_per_step": round(ms, 5), "tokens_per_s": round(cfg["n_tokens"] / (ms * 1e-3), 1),
            "steps": steps, "note": "moe_forward captured in HIP graphs and replayed"}


def gemm_roofline(cfg, name, R, live, gemm_ms):
    """The expert GEMM's roofline object (algorithmic work per launch over the average launch
    time of its two launches)."""
    N, M, H = cfg["n_tokens"], cfg["d_model"], cfg["d_ff"]
    Es = cfg["n_shared"]
    b = 2 if cfg["dtype"] == 1 else 4
    gl = 2 if cfg["act"] == configs.ACT_SWIGLU else 1
    flops_g2 = 2.0 * R * M * H + 2.0 * N * Es * H * M
    flops_launch = (gl * flops_g2 + flops_g2) / 2.0
    bytes_g1 = (R * M + gl * live * H * M + R * H +
                (N * M + gl * Es * H * M + N * Es * H if Es else 0)) * b
    bytes_g2 = (R * H + live * M * H + R * M + (N * Es * H + Es * M * H + N * M if Es else 0)) * b
    bytes_launch = (bytes_g1 + bytes_g2) / 2.0
    peak = PEAK_BF16_TFLOPS if cfg["dtype"] == 1 else PEAK_FP32_TFLOPS
    tflops = flops_launch / (gemm_ms * 1e-3) / 1e12
    gbps = bytes_launch / (gemm_ms * 1e-3) / 1e9
    bound = FFN_BOUND.get(name, "mfma")
    if bound == "mfma":
        ro = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
              "frac": round(tflops / peak, 4)}
    else:
        ro = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    ro.update({"traffic": load_traffic(name),
               "kernel": "gemm_bf16_kernel (expert GEMM 1 + act, expert GEMM 2)"
               if cfg["dtype"] == 1 else "gemm_f32_kernel (expert GEMM 1 + act, expert GEMM 2)",
               "flops_per_launch": flops_launch, "alg_bytes_per_launch": int(bytes_launch),
               "avg_launch_ms": round(gemm_ms, 5),
               "mfma_tflops": round(tflops, 2), "mfma_frac": round(tflops / peak, 4),
               "hbm_GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
               "roofline_ms": round(max(flops_launch / (peak * 1e12),
                                        bytes_launch / (PEAK_HBM_GBPS * 1e9)) * 1e3, 5)})
    return ro


def memory_kernels(cfg, R, stats, stage_avg):
    """Algorithmic bytes, GB/s and HBM fraction of the router, combine, dispatch and scan."""
    N, M, E, Es, k = (cfg[f] for f in ("n_tokens", "d_model", "n_experts", "n_shared", "top_k"))
    b = 2 if cfg["dtype"] == 1 else 4
    bytes_router = N * (M * b + 4 * E + 9 * k + (4 if cfg["random_routing"] else 0))
    bytes_combine = (R + N * int(cfg["residual"]) + N * int(Es > 0) + N) * M * b + N * k * 8
    hbm = {}
    for name, by in (("router", bytes_router), ("combine", bytes_combine)):
        t = stage_avg[name]
        gbps = by / (t * 1e-3) / 1e9
        hbm[name] = {"bytes": int(by), "ms": round(t, 5), "GB/s": round(gbps, 1),
                     "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    # Metadata kernels (64-token router blocks, nbg per group).  Capacity scan: per (g, e) it
    # reads the k rank histograms, the probability sums (fp64) and selection counts of every
    # router block and writes the k per-block bases, count, the rank totals, P and c.
    # Dispatch (forward): per slot it reads the expert id, the active flag and the gate weight
    # and writes pos, row and the weight (zero when dropped); per kept row the row->token
    # index; per router block its rank bases; the count table once.
    G = cfg["n_groups"]
    nbg = -(-(N // G) // 64)
    bytes_gate = G * E * (8 * k * nbg + 12 * nbg + 4 * k + 16)
    bytes_permute = N * k * 21 + 4 * R + 4 * G * k * E * nbg + 4 * G * E
    for name, by, note in (
            ("permute", bytes_permute, "positions, rows and the row->token index only (GEMM 1 "
                                       "gathers the token rows from x); latency-bound"),
            ("gate", bytes_gate, "capacity scan over the router blocks' histograms; "
                                 "latency-bound")):
        t = stage_avg[name]
        gbps = by / (t * 1e-3) / 1e9
        hbm[name] = {"bytes": int(by), "ms": round(t, 5), "GB/s": round(gbps, 1),
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "note": note}
    return hbm


def measure(name, args, ev, headline):
    """Time one workload; returns its result object (the headline's carries graph and the
    full CPU baseline)."""
    import torch
    cfg = configs.WORKLOADS[name]
    print(f"[bench] {name}: inputs", file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg)

    def up(n):
        bits = getattr(inp, n + "_bits")
        if bits is not None:
            return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(getattr(inp, n)).cuda()
    x0, Wg, W1, W2 = up("x"), up("Wg"), up("W1"), up("W2")
    bg = torch.from_numpy(inp.bg).cuda() if inp.bg is not None else None
    u = torch.from_numpy(inp.u).cuda() if inp.u is not None else None
    xs = [x0] + [x0.clone() for _ in range(args.copies - 1)]
    ys = [torch.empty_like(x0) for _ in range(args.copies)]
    meta = binding.alloc_meta(cfg)
    ws = binding.alloc_workspace(cfg)
    aux = torch.empty(4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    events = [ev.create(binding.MOE_N_EVENTS) for _ in range(K)]
    warm = ev.create(binding.MOE_N_EVENTS)
    lib = binding.load_library()
    cfg_c = binding.make_cfg(cfg)

    def step(i, evs):
        c = i % args.copies
        arr = (ctypes.c_void_p * binding.MOE_N_EVENTS)(*[e.value for e in evs])
        m = meta.as_struct()
        rc = lib.moe_forward_timed(
            ctypes.byref(cfg_c), xs[c].data_ptr(), Wg.data_ptr(),
            bg.data_ptr() if bg is not None else None, W1.data_ptr(), W2.data_ptr(),
            u.data_ptr() if u is not None else None, ys[c].data_ptr(), aux.data_ptr(),
            ctypes.byref(m), ws.data_ptr(), ws.numel(), stream.cuda_stream, arr)
        if rc:
            raise binding.MoeError(rc, "moe_forward_timed")

    print(f"[bench] {name}: {W} warm-up + {K} timed steps", file=sys.stderr, flush=True)
    for i in range(W):
        step(i, warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, events[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / K

    step_ms = [ev.elapsed(evs[0], evs[-1]) for evs in events]
    stage_ms = {s: [ev.elapsed(evs[si], evs[si + 1]) for evs in events]
                for si, s in enumerate(binding.STAGES)}
    ev.destroy([e for evs in events for e in evs] + warm)
    med = float(np.median(step_ms))
    stage_avg = {s: float(np.mean(v)) for s, v in stage_ms.items()}
    stats = meta.stats.cpu().numpy().astype(np.int64)
    R = int(stats[0])
    count = meta.count.cpu().numpy()
    live = int((count.sum(axis=0) > 0).sum())
    N = cfg["n_tokens"]
    gemm_ms = (stage_avg["ffn1"] + stage_avg["ffn2"]) / 2.0
    out = {
        "tokens_per_s": round(N / (med * 1e-3), 1),
        "ms_per_step": round(med, 5),
        "timing": {"median_ms": round(med, 5), "mean_ms": round(float(np.mean(step_ms)), 5),
                   "min_ms": round(float(np.min(step_ms)), 5),
                   "max_ms": round(float(np.max(step_ms)), 5), "wall_ms_per_step": round(wall_ms, 5),
                   "note": "per-step HIP events from the first launch to the last (median); "
                           "wall: K steps between two synchronisations"},
        "dtype": "bf16" if cfg["dtype"] == 1 else "f32",
        "config": {"workload": name, "n_tokens": N, "n_groups": cfg["n_groups"],
                   "d_model": cfg["d_model"], "d_ff": cfg["d_ff"], "n_experts": cfg["n_experts"],
                   "n_shared": cfg["n_shared"], "top_k": cfg["top_k"],
                   "capacity": cfg["capacity"], "random_routing": cfg["random_routing"],
                   "act": ["relu", "gelu", "swiglu"][cfg["act"]], "parallelism": "single-gpu"},
        "roofline": gemm_roofline(cfg, name, R, live, gemm_ms),
        "hbm": memory_kernels(cfg, R, stats, stage_avg),
        "stages_ms": {s: round(v, 5) for s, v in stage_avg.items()},
        "stages_median_ms": {s: round(float(np.median(v)), 5) for s, v in stage_ms.items()},
        "kept_rows": R,
        "stats": stats.tolist(),
        "aux_loss": float(aux[0].cpu()),
    }
    if headline and args.graph_steps > 0:
        print(f"[bench] {name}: graph replay", file=sys.stderr, flush=True)
        out["graph"] = graph_timing(cfg, xs, ys, Wg, bg, W1, W2, u, aux, meta, ws,
                                    args.graph_steps)
    del xs, ys, ws
    torch.cuda.empty_cache()
    if args.backward_steps > 0:
        print(f"[bench] {name}: backward", file=sys.stderr, flush=True)
        out["backward"] = backward_timing(cfg, x0, Wg, W1, W2, bg, u, R, args.backward_steps)
    del x0, Wg, W1, W2, meta
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print(f"[bench] {name}: CPU oracle baseline", file=sys.stderr, flush=True)
        # FFN sample sized to about budget flops per pass (fp64 oracle)
        budget = 2e11 if headline else 5e10
        ns = int(max(64, min(N, budget // ffn_flops_per_token(cfg))))
        out["cpu_baseline"] = cpu_baseline(cfg, inp, ns, min_seconds=10.0 if headline else 3.0)
    del inp
    return out


def library_gemm_timing(reps=10):
    """torch.matmul in bf16 (contiguous operands, so the library sees plain row-major GEMMs) on
    the large-expert layer's two GEMMs as dense problems (32768 rows = 16384 tokens x top-2)
    and on GShard's two expert GEMMs as a batch of 64 experts padded to 512 rows each (its mean
    of 16384 x 2 / 64 rows, so no expert is dropped only if the routing is exactly even).  The
    median of reps launches, timed with events on torch's current stream."""
    import torch
    shapes = {
        "large_expert_gemm1_dense": (1, 32768, 4096, 14336),
        "large_expert_gemm2_dense": (1, 32768, 14336, 4096),
        "gshard_gemm1_batched_padded": (64, 512, 1024, 4096),
        "gshard_gemm2_batched_padded": (64, 512, 4096, 1024),
    }
    try:
        blas = str(torch.backends.cuda.preferred_blas_library())
    except Exception:   # older torch: the library choice is not exposed
        blas = "default"
    res = {"blas": blas, "torch": torch.__version__}
    g = torch.Generator(device="cuda").manual_seed(7)
    for name, (b, m, k, n) in shapes.items():
        a = torch.randn(b, m, k, device="cuda", dtype=torch.bfloat16, generator=g)
        w = torch.randn(b, k, n, device="cuda", dtype=torch.bfloat16, generator=g).contiguous()
        if b == 1:
            a, w = a[0], w[0]
        c = torch.matmul(a, w)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, w, out=c)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        tf = 2.0 * b * m * k * n / (ms * 1e-3) / 1e12
        res[name] = {"shape": [b, m, k, n], "ms": round(ms, 4), "TFLOPs": round(tf, 1),
                     "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 3)}
        del a, w, c
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(configs.WORKLOADS),
                    help="the headline layer")
    ap.add_argument("--configs", default=",".join(OTHER_CONFIGS),
                    help="other layers measured in the same run (comma-separated, or 'none')")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copies", type=int, default=4, help="rotating copies of x and y")
    ap.add_argument("--graph-steps", type=int, default=50,
                    help="headline forward steps replayed from HIP graphs (0: skip)")
    ap.add_argument("--backward-steps", type=int, default=10,
                    help="timed moe_backward calls per layer (0: skip)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch's bf16 matmul (the ROCm BLAS library) on the dense "
                         "large-expert GEMM shapes and on GShard's expert GEMMs padded to 512 "
                         "rows per expert, for comparison with the expert GEMM")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 3 device-to-device copies of 1 GiB (the known-size kernel "
                         "that scales the HBM byte counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs the MoE layer on exactly one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported: the layer has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    others = [] if args.configs in ("", "none") else args.configs.split(",")
    for o in others:
        if o not in configs.WORKLOADS:
            print(f"unknown workload {o}", file=sys.stderr)
            sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.int32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel() * 4, "launches": 3}))
        return
    binding.load_library()
    ev = HipEvents()
    head = measure(args.workload, args, ev, headline=True)

    # Achievable copy bandwidth in the same run (1 GiB device-to-device clone).
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    tc0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 2 * 5 / (time.perf_counter() - tc0) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    rest = {}
    for o in others:
        if o != args.workload:
            rest[o] = measure(o, args, ev, headline=False)

    out = {
        "metric": "MoE layer fwd tokens/s on 1 GPU + expert-GEMM % bf16 MFMA peak + HBM % peak",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded x ~ N(0,1), weights ~ N(0, 1/fan_in), random-init experts)",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "timing": head["timing"],
        "hbm": head["hbm"],
        "copy_GBps": round(copy_gbps, 1),
        "stages_ms": head["stages_ms"],
        "stages_median_ms": head["stages_median_ms"],
        "kept_rows": head["kept_rows"],
        "stats": head["stats"],
        "aux_loss": head["aux_loss"],
    }
    for key in ("graph", "backward"):
        if key in head:
            out[key] = head[key]
    if args.library_gemm:
        out["library_gemm"] = library_gemm_timing()
    if out["cpu_baseline"] is None:
        del out["cpu_baseline"]
    out["configs"] = rest
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
