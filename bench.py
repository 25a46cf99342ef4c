"""Benchmark of the single-GPU MoE layer forward (HIP path) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one full moe_forward (router, capacity scan, dispatch, expert GEMM 1 + act,
expert GEMM 2, combine + aux) over one batch of seeded synthetic tokens already resident in
HBM.  W untimed steps, then K timed steps bracketed by torch.cuda.synchronize(); HIP events
recorded by the library at the stage boundaries (on the launch stream) give per-stage
times.  Prints one JSON line.

The roofline object is for the dominant kernel, the expert GEMM: algorithmic flops per
launch (2 R M H for the routed rows, + 2 N Es H M for shared experts; R = kept rows) over
the average launch time of its two launches per step, against the bf16 dense MFMA peak.
The cpu_baseline object times the CPU oracle on a bounded sample of the same workload.
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


def cpu_baseline(cfg, inp, logits32, budget_tokens):
    """Time the CPU oracle: routing + aux over all N tokens, FFN + combine over a sample."""
    from oracle import moe_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas_threads = 1
    N = cfg["n_tokens"]
    t0 = time.perf_counter()
    logits = mo.router_logits(inp.x, inp.Wg, inp.bg)
    r = mo.route(cfg, logits.astype(np.float32), inp.u)
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng(1)
    ns = min(N, budget_tokens)
    toks = np.sort(rng.choice(N, size=ns, replace=False))
    t0 = time.perf_counter()
    mo.layer_outputs(cfg, inp.x, inp.W1, inp.W2, r, tokens=toks)
    t_ffn = time.perf_counter() - t0
    per_token = t_route / N + t_ffn / ns
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": (f"float64 NumPy oracle: router logits + routing + positions + aux over "
                       f"all {N} tokens ({t_route:.2f} s), expert FFN + combine over a seeded "
                       f"sample of {ns} tokens ({t_ffn:.2f} s); tokens/s = 1 / (route s/token "
                       f"+ FFN s/token); host os.cpu_count()={os.cpu_count()}, BLAS threads="
                       f"{blas_threads}")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=configs.BENCH_WORKLOAD, choices=sorted(configs.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=16384)
    ap.add_argument("--copies", type=int, default=4, help="rotating copies of x and y")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs the MoE layer on exactly one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE={world}) is not supported by this build", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
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

    # Dominant kernel: the expert GEMM (two launches per step with equal flops).
    flops_launch = 2.0 * R * M * H + 2.0 * N * Es * H * M
    gemm_ms = (stage_avg["ffn1"] + stage_avg["ffn2"]) / 2.0
    achieved = flops_launch / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg["dtype"] == 1 else PEAK_FP32_TFLOPS
    traffic = load_traffic(args.workload, flops_launch)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
                "kernel": "gemm_bf16_kernel (expert GEMM 1 and 2)",
                "flops_per_launch": flops_launch, "avg_launch_ms": round(gemm_ms, 5)}

    # Memory-bound kernels: algorithmic bytes / time against the HBM peak.
    kept_tokens = N - int(stats[2])
    bytes_router = N * (M * b + 4 * E + 9 * k + (4 if cfg["random_routing"] else 0))
    bytes_permute = kept_tokens * M * b + R * M * b + N * k * 13
    bytes_combine = (R + N * int(cfg["residual"]) + N * int(Es > 0) + N) * M * b + N * k * 8
    hbm = {}
    for name, by in (("router", bytes_router), ("permute", bytes_permute),
                     ("combine", bytes_combine)):
        t = stage_avg[name]
        gbps = by / (t * 1e-3) / 1e9
        hbm[name] = {"bytes": int(by), "ms": round(t, 5), "GB/s": round(gbps, 1),
                     "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    hbm["gate"] = {"ms": round(stage_avg["gate"], 5), "note": "capacity scan + offsets; latency-bound"}

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
                   "act": ["relu", "gelu"][cfg["act"]], "parallelism": "single-gpu"},
        "roofline": roofline,
        "hbm": hbm,
        "copy_GBps": round(copy_gbps, 1),
        "stages_ms": {s: round(v, 5) for s, v in stage_avg.items()},
        "kept_rows": R,
        "stats": stats.tolist(),
        "aux_loss": float(aux[0].cpu()),
    }
    ev.destroy([e for evs in events for e in evs] + warm)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, meta.logits.cpu().numpy(), args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
