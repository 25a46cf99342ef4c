"""Seeded synthetic inputs for the MoE layer.

This module only draws numbers.  It holds none of the layer's arithmetic, and both
the HIP path (through the tests and the benchmark) and the CPU oracle consume what it
returns, so it is the one piece of code the two sides share.

Recipe (one ``numpy.random.default_rng(seed)`` stream, PCG64, drawn in this order):
  x   [N, M]            ~ N(0, 1)
  Wg  [E, M]            ~ N(0, 1/M)       (row e is expert e's gate vector)
  W1  [E+Es, H, M]      ~ N(0, 1/M)       (row n of W1[e] feeds hidden unit n;
                                           [E+Es, 2H, M] for the gated expert, act 2:
                                           H gate rows, then H up rows)
  W2  [E+Es, M, H]      ~ N(0, 1/H)       (row m of W2[e] feeds output feature m)
  u   [N]               ~ U[0, 1) fp32    (only when random routing is on)
  bg  [E]               = -s * ln(e + 1)  (only when zipf_s > 0: the log of a Zipf(s)
                                           weight of rank e+1; expert 0 is the hottest)
Shared experts are the last Es entries of W1 and W2.  Everything is drawn in fp32 and,
for bf16 layers, rounded to bf16 (round to nearest even); both sides read the rounded
values.
"""
import numpy as np


def round_to_bf16_bits(a):
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """uint16 bf16 bit patterns -> the fp32 values they encode (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng, shape, std):
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def w1_rows(cfg):
    """Rows of one expert's W1: H, or 2H (gate and up projections) for the gated expert."""
    return 2 * cfg["d_ff"] if cfg["act"] == 2 else cfg["d_ff"]


class Inputs:
    """Host copies of one layer's inputs.

    For each tensor ``t`` in x, Wg, W1, W2: ``t`` holds the fp32 values the layer sees
    (already rounded to bf16 for bf16 layers) and ``t_bits`` the uint16 bf16 encoding
    (None for fp32 layers).  ``u`` and ``bg`` are fp32 or None.
    """

    def __init__(self, cfg, seed=None):
        seed = cfg.get("seed", 0) if seed is None else seed
        rng = np.random.default_rng(seed)
        N, M, H = cfg["n_tokens"], cfg["d_model"], cfg["d_ff"]
        E, Es = cfg["n_experts"], cfg["n_shared"]
        self.cfg = cfg
        self.seed = seed
        raw = {
            "x": _normal(rng, (N, M), 1.0),
            "Wg": _normal(rng, (E, M), (1.0 / M) ** 0.5),
            "W1": _normal(rng, (E + Es, w1_rows(cfg), M), (1.0 / M) ** 0.5),
            "W2": _normal(rng, (E + Es, M, H), (1.0 / H) ** 0.5),
        }
        self.u = rng.random(size=N, dtype=np.float32) if cfg["random_routing"] else None
        s = float(cfg.get("zipf_s", 0.0))
        self.bg = ((-s) * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32) \
            if s > 0 else None
        bf16 = cfg["dtype"] == 1
        for name, arr in raw.items():
            if bf16:
                bits = round_to_bf16_bits(arr)
                setattr(self, name + "_bits", bits)
                setattr(self, name, bf16_bits_to_f32(bits))
            else:
                setattr(self, name + "_bits", None)
                setattr(self, name, arr)
        del raw


def make_inputs(cfg, seed=None):
    return Inputs(cfg, seed)


def upstream_grad(cfg, seed=None):
    """Seeded upstream gradient dy [N, M] ~ N(0, 1) for the backward pass, drawn from its own
    stream (SeedSequence entropy [seed, 1]) so the forward inputs are unchanged.  Returns
    (fp32 values, bf16 bits or None), rounded like the other inputs for bf16 layers."""
    seed = cfg.get("seed", 0) if seed is None else seed
    rng = np.random.default_rng([seed, 1])
    dy = _normal(rng, (cfg["n_tokens"], cfg["d_model"]), 1.0)
    if cfg["dtype"] == 1:
        bits = round_to_bf16_bits(dy)
        return bf16_bits_to_f32(bits), bits
    return dy, None
