"""Reference router-side gradients of bf16 layers (dWg, dbg), shared by the GPU backward tests
and the CPU tests that pin it.

The combine weights' gradient dw_nj = <dy_n W2_e, h_row> is formed on the device from the
hidden activation h and the product dy W2_e, both in the layer's dtype (the layer keeps its
hidden activations in bf16; the oracle rounds nothing).  dWg and dbg are linear in dw, and
where a few tokens dominate them their dw terms cancel, so the rounding of h alone can move
them by more than the relative tolerance.  For bf16 layers they are therefore compared with the
oracle's router chain (oracle.moe_backward.router_backward) fed the dw of bf16-rounded h and
dy W2_e, formed here from the oracle's own float64 activations: the rounding is the layer's,
every other step the oracle's.
"""
import numpy as np

from mixture_experts_layer_group_amd import synth
from oracle import moe_backward as mb
from oracle import moe_oracle as mo


def _bf16(a):
    return synth.bf16_bits_to_f32(synth.round_to_bf16_bits(np.asarray(a, np.float32))).astype(
        np.float64)


def dw_of(cfg, inp, r, dy, rounded=True):
    """[N, k] combine weights' gradient of the kept slots (0 elsewhere), from h and dy W2_e
    rounded to bf16 (or exact with rounded=False)."""
    N, k, E = cfg["n_tokens"], cfg["top_k"], cfg["n_experts"]
    rnd = _bf16 if rounded else (lambda a: a)
    dw = np.zeros((N, k))
    x = np.asarray(inp.x, np.float64)
    dy = np.asarray(dy, np.float64)
    kept = r["pos"] >= 0
    for e in range(E):
        w1 = np.asarray(inp.W1[e], np.float64)
        w2 = np.asarray(inp.W2[e], np.float64)
        for j in range(k):
            rows = np.nonzero(kept[:, j] & (r["topk_idx"][:, j] == e))[0]
            if rows.size == 0:
                continue
            z = x[rows] @ w1.T
            if cfg["act"] == mo.ACT_SWIGLU:
                H = w1.shape[0] // 2
                h = mo.swish(z[:, :H]) * z[:, H:]
            else:
                h = mo.activation(z, cfg["act"])
            dw[rows, j] = (rnd(dy[rows] @ w2) * rnd(h)).sum(axis=1)
    return dw


def router_grads(cfg, inp, r, dy, logits, coefs, rounded=True):
    """(dWg, dbg, dl) of the oracle's router chain on dw_of(..., rounded)."""
    lr = np.asarray(logits, np.float32).astype(np.float64)
    dl = mb.router_backward(cfg, r["p"], r["topk_idx"], lr, dw_of(cfg, inp, r, dy, rounded),
                            **coefs)
    return dl.T @ np.asarray(inp.x, np.float64), dl.sum(axis=0), dl
