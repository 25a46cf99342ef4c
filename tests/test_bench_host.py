"""Host-side behaviour of bench.py (no GPU): the one-GPU refusal, the missing-GPU error, the
CPU-oracle baseline object and the kernel-source hash that gates the committed HBM traffic."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_layer_group_amd import configs, synth  # noqa: E402


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=e, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("args,env", [(("--gpus", "2"), None), ((), {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(args, env):
    p = _run(*args, env=env)
    assert p.returncode == 2
    assert "exactly one GPU" in p.stderr
    assert p.stdout == ""


@pytest.mark.parametrize("extra", [(), ("--library-gemm",)])
def test_no_gpu_is_an_error_not_a_fallback(extra):
    """Also with the library comparison asked for: nothing runs on the CPU in its place."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    p = _run("--steps", "1", "--warmup", "0", *extra)
    assert p.returncode == 1
    assert "needs a GPU" in p.stderr
    assert p.stdout == ""


def test_cpu_baseline_object():
    cfg = configs.WORKLOADS["tiny_fp32"]
    inp = synth.make_inputs(cfg)
    cb = bench.cpu_baseline(cfg, inp, budget_tokens=64, min_seconds=0.0, max_passes=2)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "64 tokens" in cb["sample"] and "all 256 tokens" in cb["sample"]
    json.dumps(cb)


def test_traffic_is_only_reported_for_the_profiled_kernel_source():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    for wl, rec in t["workloads"].items():
        if t["kernel_hash"] == bench.kernel_hash():
            assert bench.load_traffic(wl) == rec["hbm_bytes_per_launch"]
        else:
            assert bench.load_traffic(wl) is None
    other = next(w for w in configs.WORKLOADS if w not in t["workloads"])
    assert bench.load_traffic(other) is None


def test_cpu_baseline_names_the_host_cpu():
    cfg = configs.WORKLOADS["tiny_fp32"]
    inp = synth.make_inputs(cfg)
    cb = bench.cpu_baseline(cfg, inp, budget_tokens=32, min_seconds=0.0, max_passes=1)
    assert bench.cpu_model() in cb["sample"] and "os.cpu_count()" in cb["sample"]


def test_roofline_bound_follows_the_layer_shapes():
    """MFMA for the contractions, HBM for the weight-streaming Switch-style layer; frac is the
    fraction against that bound's peak."""
    for name in ("gshard_bf16", "large_expert_bf16", "shared_routed_bf16", "switch_bf16"):
        cfg = configs.WORKLOADS[name]
        ro = bench.gemm_roofline(cfg, name, R=cfg["n_tokens"], live=cfg["n_experts"],
                                 gemm_ms=1.0)
        want = "hbm" if name == "switch_bf16" else "mfma"
        assert ro["bound"] == want
        frac = ro["hbm_frac"] if want == "hbm" else ro["mfma_frac"]
        assert ro["frac"] == frac and ro["peak"] == (bench.PEAK_HBM_GBPS if want == "hbm"
                                                     else bench.PEAK_BF16_TFLOPS)
