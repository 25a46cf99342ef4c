"""Seeded synthetic inputs for the MoE layer.

This module only draws numbers.  It holds none of the layer's arithmetic, and both
the HIP path (through the tests and the benchmark) and the CPU oracle consume what it
returns, so it is the one piece of code the two sides share.

Recipe.  Every tensor is drawn in fixed chunks of 2^22 consecutive elements (row-major order),
chunk c of tensor t from its own stream ``numpy.random.default_rng([seed, t, c])`` (PCG64
seeded through SeedSequence), so chunks can be drawn in parallel and the values do not depend
on the number of threads.  Tensor ids t:
  0 x   [N, M]            ~ N(0, 1)
  1 Wg  [E, M]            ~ N(0, 1/M)       (row e is expert e's gate vector)
  2 W1  [E+Es, H, M]      ~ N(0, 1/M)       (row n of W1[e] feeds hidden unit n;
                                             [E+Es, 2H, M] for the gated expert, act 2:
                                             H gate rows, then H up rows)
  3 W2  [E+Es, M, H]      ~ N(0, 1/H)       (row m of W2[e] feeds output feature m)
  4 u   [N]               ~ U[0, 1) fp32    (only when random routing is on)
  5 dy  [N, M]            ~ N(0, 1)         (the backward's upstream gradient)
    bg  [E]               = -s * ln(e + 1)  (only when zipf_s > 0: the log of a Zipf(s)
                                             weight of rank e+1; expert 0 is the hottest)
Shared experts are the last Es entries of W1 and W2.  Everything is drawn in fp32 and,
for bf16 layers, rounded to bf16 (round to nearest even); both sides read the rounded
values.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22          # elements per independently seeded chunk
T_X, T_WG, T_W1, T_W2, T_U, T_DY = range(6)


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(total, fill):
    """Run fill(c, lo, hi) over the chunks [lo, hi) of [0, total), in parallel threads (NumPy's
    generators and ufuncs release the GIL on large arrays)."""
    n = (total + CHUNK - 1) // CHUNK
    if n <= 1:
        for c in range(n):
            fill(c, 0, total)
        return
    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(lambda c: fill(c, c * CHUNK, min(total, (c + 1) * CHUNK)), range(n)))


def _round_chunk(flat_in, flat_out, lo, hi):
    bits = flat_in[lo:hi].view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    flat_out[lo:hi] = (bits + rounding) >> np.uint32(16)


def round_to_bf16_bits(a):
    """fp32 array -> uint16 bf16 bit patterns, round to nearest even (finite inputs)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    fa, fo = a.reshape(-1), out.reshape(-1)
    _chunked(fa.size, lambda c, lo, hi: _round_chunk(fa, fo, lo, hi))
    return out


def bf16_bits_to_f32(b):
    """uint16 bf16 bit patterns -> the fp32 values they encode (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.uint32)
    fb, fo = b.reshape(-1), out.reshape(-1)

    def fill(c, lo, hi):
        fo[lo:hi] = fb[lo:hi].astype(np.uint32) << np.uint32(16)
    _chunked(fb.size, fill)
    return out.view(np.float32)


def _normal(seed, tid, shape, std):
    """N(0, std^2) fp32 of the given shape, chunk c drawn from default_rng([seed, tid, c])."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)

    def fill(c, lo, hi):
        np.random.default_rng([seed, tid, c]).standard_normal(
            size=hi - lo, dtype=np.float32, out=flat[lo:hi])
        if std != 1.0:
            flat[lo:hi] *= np.float32(std)
    _chunked(flat.size, fill)
    return out


def _uniform(seed, tid, n):
    """U[0, 1) fp32, chunked like _normal."""
    out = np.empty(n, dtype=np.float32)

    def fill(c, lo, hi):
        np.random.default_rng([seed, tid, c]).random(size=hi - lo, dtype=np.float32,
                                                     out=out[lo:hi])
    _chunked(n, fill)
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
        N, M, H = cfg["n_tokens"], cfg["d_model"], cfg["d_ff"]
        E, Es = cfg["n_experts"], cfg["n_shared"]
        self.cfg = cfg
        self.seed = seed
        raw = {
            "x": _normal(seed, T_X, (N, M), 1.0),
            "Wg": _normal(seed, T_WG, (E, M), (1.0 / M) ** 0.5),
            "W1": _normal(seed, T_W1, (E + Es, w1_rows(cfg), M), (1.0 / M) ** 0.5),
            "W2": _normal(seed, T_W2, (E + Es, M, H), (1.0 / H) ** 0.5),
        }
        self.u = _uniform(seed, T_U, N) if cfg["random_routing"] else None
        s = float(cfg.get("zipf_s", 0.0))
        self.bg = ((-s) * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32) \
            if s > 0 else None
        bf16 = cfg["dtype"] == 1
        for name in list(raw):
            arr = raw.pop(name)
            if bf16:
                bits = round_to_bf16_bits(arr)
                del arr
                setattr(self, name + "_bits", bits)
                setattr(self, name, bf16_bits_to_f32(bits))
            else:
                setattr(self, name + "_bits", None)
                setattr(self, name, arr)


def make_inputs(cfg, seed=None):
    return Inputs(cfg, seed)


def upstream_grad(cfg, seed=None):
    """Seeded upstream gradient dy [N, M] ~ N(0, 1) for the backward pass (tensor id 5, so the
    forward inputs are unchanged).  Returns (fp32 values, bf16 bits or None), rounded like the
    other inputs for bf16 layers."""
    seed = cfg.get("seed", 0) if seed is None else seed
    dy = _normal(seed, T_DY, (cfg["n_tokens"], cfg["d_model"]), 1.0)
    if cfg["dtype"] == 1:
        bits = round_to_bf16_bits(dy)
        return bf16_bits_to_f32(bits), bits
    return dy, None
