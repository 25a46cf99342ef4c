"""Seeded random layer configurations for the parity sweep (tests/test_gpu_random_layers.py).

Every option of the layer is drawn: dtype, model and hidden widths, expert count, top-k,
group-limited routing, random routing, capacity from a fifth of the balanced load to well
above it, activation, gate normalisation, shared experts, residual, and the router-offset
skew.  Sizes stay small enough for the fp64 oracle to run each case in well under a second.
"""
import numpy as np

from mixture_experts_layer_group_amd import configs

N_CASES = 24


def random_cfg(i):
    r = np.random.default_rng(7000 + i)
    dtype = configs.DTYPE_BF16 if r.random() < 0.75 else configs.DTYPE_F32
    mul = 128 if dtype == configs.DTYPE_BF16 else 64
    M = mul * int(r.integers(1, 4))
    H = mul * int(r.integers(1, 5))
    E = int(r.choice([1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32, 64]))
    eg = int(r.choice([d for d in (1, 2, 4, 8) if E % d == 0]))
    tg = int(r.integers(1, eg + 1))
    k = int(r.integers(1, min(8, tg * (E // eg)) + 1))
    rr = int(k == 2 and r.random() < 0.3)
    G = int(r.choice([1, 2, 3, 4]))
    S = int(r.integers(1, 700))
    C = max(1, int(round(r.uniform(0.2, 2.5) * k * S / E)))
    return configs._cfg(
        f"random_{i}", n_tokens=G * S, n_groups=G, d_model=M, d_ff=H, n_experts=E, top_k=k,
        capacity=C, act=int(r.integers(0, 3)), gate_norm=int(r.integers(0, 3)), dtype=dtype,
        n_shared=int(r.choice([0, 0, 1, 2])), random_routing=rr,
        residual=int(r.random() < 0.8), norm_p=float(r.choice([0.5, 1.0, 2.0, 3.0])),
        expert_groups=eg, topk_groups=tg, zipf_s=float(r.choice([0.0, 0.0, 0.8, 1.3])),
        seed=300 + i)


CASES = [random_cfg(i) for i in range(N_CASES)]
