"""Benchmark of the single-GPU MoE layer forward (HIP path) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one full moe_forward (router, capacity scan, dispatch, expert GEMM 1 + act,
expert GEMM 2, combine + aux) over one batch of seeded synthetic tokens already resident in
HBM.  W untimed steps, then K timed steps bracketed by torch.cuda.synchronize(); HIP events
recorded by the library at the stage boundaries (on the launch stream) give per-stage
times.  Prints one JSON line.

The roofline object is for the dominant kernel, the expert GEMM: algorithmic flops per
launch (2 R M H for the routed rows, + 2 N Es H M for shared experts; R = kept rows; the
gated experts' GEMM 1 does twice that) averaged over its two launches per step, over their
average launch time, against the bf16 dense MFMA peak.
The cpu_baseline object times the CPU oracle on a bounded sample of the same workload.
The graph object replays the same step from HIP graphs (no host launch work between the
kernels); the backward object times moe_backward (routing and activations recomputed).
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
    for f in ("moe_expert_ffn.hip", "moe_device.h", "moe_internal.h"):
        with open(os.path.join(ROOT, "mixture_experts_layer_group_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, flops_per_launch):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, or None when
    the counters were taken on another kernel version or workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, inp, budget_tokens, min_seconds=10.0, max_passes=20):
    """Time the CPU oracle as it stands: router logits + routing + positions + aux over all N
    tokens, expert FFN + combine over a seeded sample, repeated until ~min_seconds of CPU work
    has been timed."""
    from oracle import moe_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas_threads = 1
    N = cfg["n_tokens"]
    ns = min(N, budget_tokens)
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
                       f"s/token); host os.cpu_count()={os.cpu_count()}, BLAS threads="
                       f"{blas_threads}")}


def backward_timing(cfg, inp, x, Wg, W1, W2, bg, u, R, steps):
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        binding.moe_backward(cfg, x, Wg, bg, W1, W2, u, dy, coefs["coef_aux"], coefs["coef_z"],
                             coefs["coef_dev"], out["dx"], out["dWg"], out["dbg"], out["dW1"],
                             out["dW2"], meta, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    N, M, H, Es = cfg["n_tokens"], cfg["d_model"], cfg["d_ff"], cfg["n_shared"]
    gl = 2 if cfg["act"] == configs.ACT_SWIGLU else 1
    fwd_ffn = (gl + 1) * 2.0 * M * H * (R + N * Es)
    recompute = gl * 2.0 * M * H * (R + N * Es)
    return {"ms": round(ms, 4), "tokens_per_s": round(N / (ms * 1e-3), 1), "steps": steps,
            "ffn_flops_backward": 2 * fwd_ffn, "ffn_flops_recompute": recompute,
            "tflops_backward_alg": round(2 * fwd_ffn / (ms * 1e-3) / 1e12, 2),
            "tflops_incl_recompute": round((2 * fwd_ffn + recompute) / (ms * 1e-3) / 1e12, 2),
            "workspace_bytes": ws.numel()}


def graph_timing(cfg, xs, ys, Wg, bg, W1, W2, u, aux, meta, ws, steps):
    """The same forward step replayed from HIP graphs (one captured moe_forward per rotating
    x/y copy), which removes the host launch work between the five kernels."""
    import torch
    from mixture_experts_layer_group_amd import binding
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=configs.BENCH_WORKLOAD, choices=sorted(configs.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=16384)
    ap.add_argument("--copies", type=int, default=4, help="rotating copies of x and y")
    ap.add_argument("--graph-steps", type=int, default=50,
                    help="forward steps replayed from HIP graphs, reported beside the eager "
                         "timing (0: skip)")
    ap.add_argument("--backward-steps", type=int, default=10,
                    help="timed moe_backward calls reported beside the forward (0: skip)")
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
    cfg = configs.WORKLOADS[args.workload]
    inp = synth.make_inputs(cfg)
    dt = binding.torch_dtype(cfg)

    def up(name):
        bits = getattr(inp, name + "_bits")
        if bits is not None:
            return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(getattr(inp, name)).cuda()
    x0, Wg, W1, W2 = up("x"), up("Wg"), up("W1"), up("W2")
    bg = torch.from_numpy(inp.bg).cuda() if inp.bg is not None else None
    u = torch.from_numpy(inp.u).cuda() if inp.u is not None else None
    xs = [x0] + [x0.clone() for _ in range(args.copies - 1)]
    ys = [torch.empty_like(x0) for _ in range(args.copies)]
    meta = binding.alloc_meta(cfg)
    ws = binding.alloc_workspace(cfg)
    aux = torch.empty(4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    ev = HipEvents()
    K, W = args.steps, args.warmup
    events = [ev.create(binding.MOE_N_EVENTS) for _ in range(K)]
    warm = ev.create(binding.MOE_N_EVENTS)

    def step(i, evs):
        c = i % args.copies
        arr = (ctypes.c_void_p * binding.MOE_N_EVENTS)(*[e.value for e in evs])
        m = meta.as_struct()
        rc = binding.load_library().moe_forward_timed(
            ctypes.byref(binding.make_cfg(cfg)), xs[c].data_ptr(), Wg.data_ptr(),
            bg.data_ptr() if bg is not None else None, W1.data_ptr(), W2.data_ptr(),
            u.data_ptr() if u is not None else None, ys[c].data_ptr(), aux.data_ptr(),
            ctypes.byref(m), ws.data_ptr(), ws.numel(), stream.cuda_stream, arr)
        if rc:
            raise binding.MoeError(rc, "moe_forward_timed")

    for i in range(W):
        step(i, warm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    stage_ms = {s: [] for s in binding.STAGES}
    for evs in events:
        for si, s in enumerate(binding.STAGES):
            stage_ms[s].append(ev.elapsed(evs[si], evs[si + 1]))
    stage_avg = {s: float(np.mean(v)) for s, v in stage_ms.items()}
    stats = meta.stats.cpu().numpy().astype(np.int64)
    R = int(stats[0])
    N, M, H = cfg["n_tokens"], cfg["d_model"], cfg["d_ff"]
    E, Es, k = cfg["n_experts"], cfg["n_shared"], cfg["top_k"]
    b = 2 if cfg["dtype"] == 1 else 4

    # Dominant kernel: the expert GEMM (two launches per step: GEMM 1 with the activation and
    # GEMM 2, two instantiations of gemm_bf16_kernel).  Algorithmic work per launch: flops
    # 2 R M H (+ 2 N Es H M), doubled for the gated GEMM 1 (gate and up projections); bytes =
    # the activations read and written once plus the weights of every expert that received
    # rows; both averaged over the two launches.
    count = meta.count.cpu().numpy()
    live = int((count.sum(axis=0) > 0).sum())
    gl = 2 if cfg["act"] == configs.ACT_SWIGLU else 1
    flops_g2 = 2.0 * R * M * H + 2.0 * N * Es * H * M
    flops_launch = (gl * flops_g2 + flops_g2) / 2.0
    bytes_g1 = (R * M + gl * live * H * M + R * H +
                (N * M + gl * Es * H * M + N * Es * H if Es else 0)) * b
    bytes_g2 = (R * H + live * M * H + R * M + (N * Es * H + Es * M * H + N * M if Es else 0)) * b
    bytes_launch = (bytes_g1 + bytes_g2) / 2.0
    gemm_ms = (stage_avg["ffn1"] + stage_avg["ffn2"]) / 2.0
    peak = PEAK_BF16_TFLOPS if cfg["dtype"] == 1 else PEAK_FP32_TFLOPS
    tflops = flops_launch / (gemm_ms * 1e-3) / 1e12
    gbps = bytes_launch / (gemm_ms * 1e-3) / 1e9
    t_mfma = flops_launch / (peak * 1e12)
    t_hbm = bytes_launch / (PEAK_HBM_GBPS * 1e9)
    traffic = load_traffic(args.workload, flops_launch)
    if t_mfma >= t_hbm:
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(tflops / peak, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    roofline.update({"traffic": traffic,
                     "kernel": "gemm_bf16_kernel (expert GEMM 1 + act, expert GEMM 2)",
                     "flops_per_launch": flops_launch, "alg_bytes_per_launch": int(bytes_launch),
                     "avg_launch_ms": round(gemm_ms, 5),
                     "mfma_tflops": round(tflops, 2), "mfma_frac": round(tflops / peak, 4),
                     "hbm_GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "roofline_ms": round(max(t_mfma, t_hbm) * 1e3, 5)})

    # Memory-bound kernels: algorithmic bytes / time against the HBM peak.
    kept_tokens = N - int(stats[2])
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

    out = {
        "metric": "MoE layer fwd tokens/s on 1 GPU + expert-GEMM % bf16 MFMA peak + HBM % peak",
        "value": round(N / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg["dtype"] == 1 else "f32",
        "data": "synthetic (seeded x ~ N(0,1), weights ~ N(0, 1/fan_in), random-init experts)",
        "config": {"workload": args.workload, "n_tokens": N, "n_groups": cfg["n_groups"],
                   "d_model": M, "d_ff": H, "n_experts": E, "n_shared": Es, "top_k": k,
                   "capacity": cfg["capacity"], "random_routing": cfg["random_routing"],
                   "act": ["relu", "gelu", "swiglu"][cfg["act"]], "parallelism": "single-gpu"},
        "roofline": roofline,
        "hbm": hbm,
        "copy_GBps": round(copy_gbps, 1),
        "stages_ms": {s: round(v, 5) for s, v in stage_avg.items()},
        "kept_rows": R,
        "stats": stats.tolist(),
        "aux_loss": float(aux[0].cpu()),
    }
    ev.destroy([e for evs in events for e in evs] + warm)
    if args.graph_steps > 0:
        out["graph"] = graph_timing(cfg, xs, ys, Wg, bg, W1, W2, u, aux, meta, ws,
                                    args.graph_steps)
    if args.backward_steps > 0:
        out["backward"] = backward_timing(cfg, inp, x0, Wg, W1, W2, bg, u, R, args.backward_steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
