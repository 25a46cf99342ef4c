"""Acceptance bound of the ReLU layers' dW1 (shared by the GPU backward tests and the CPU test
that pins it).

ReLU' is a decision on the sign of the pre-activation z, which the GPU computes with fp32
accumulation and the oracle in fp64: where |z| is within the accumulation error of 0,
either decision is a valid result.  One (row, hidden unit) decision adds or removes the
term dh[row, h] x[row, :] of dW1[e][h][:] (dh: the gradient at the activation's output).
The dW1 check therefore accepts every combination of decisions at the pairs with an oracle
|z| < RELU_DELTA (about 1000x the GPU's accumulation error): each element of dW1 must lie
within the tolerance plus the sum of |dh| |x| over its ambiguous pairs.  No element is left
out of the comparison.
"""
import numpy as np

RELU_DELTA = 1e-4


def relu_decision_slack(cfg, inp, r, dy):
    """Elementwise bound [E + Es, H, M] on how far any choice of the ambiguous ReLU decisions
    moves dW1, and the number of ambiguous (row, hidden unit) pairs.  Zero for other
    activations."""
    E, Es = cfg["n_experts"], cfg["n_shared"]
    slack = np.zeros(np.shape(inp.W1))
    if cfg["act"] != 0:
        return slack, 0
    x = np.asarray(inp.x, np.float64)
    dy = np.asarray(dy, np.float64)
    kept = r["pos"] >= 0
    n_amb = 0

    def add(e, rows, do):
        nonlocal n_amb
        z = x[rows] @ np.asarray(inp.W1[e], np.float64).T
        amb = np.abs(z) < RELU_DELTA
        n_amb += int(amb.sum())
        if amb.any():
            dh = do @ np.asarray(inp.W2[e], np.float64)
            slack[e] += (np.abs(dh) * amb).T @ np.abs(x[rows])

    for e in range(E):
        for j in range(cfg["top_k"]):
            rows = np.nonzero(kept[:, j] & (r["topk_idx"][:, j] == e))[0]
            if rows.size:
                add(e, rows, r["topk_w"][rows, j][:, None] * dy[rows])
    for q in range(Es):
        add(E + q, np.arange(cfg["n_tokens"]), dy)
    return slack, n_amb
