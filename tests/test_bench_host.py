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


def test_no_gpu_is_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    p = _run("--steps", "1", "--warmup", "0")
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
    wl = t["workload"]
    if t["kernel_hash"] == bench.kernel_hash():
        assert bench.load_traffic(wl, 1.0) == t["hbm_bytes_per_launch"]
    else:
        assert bench.load_traffic(wl, 1.0) is None
    other = next(w for w in configs.WORKLOADS if w != wl)
    assert bench.load_traffic(other, 1.0) is None
