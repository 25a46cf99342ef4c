"""Acceptance bounds of the ReLU layers' dW1 and dx (shared by the GPU backward tests and the
CPU tests that pin them).

ReLU' is a decision on the sign of the pre-activation z, which the GPU computes with fp32
accumulation and the oracle in fp64: where |z| is within the accumulation error of 0,
either decision is a valid result.  One (row, hidden unit) decision adds or removes the
term dh[row, h] x[row, :] of dW1[e][h][:] (dh: the gradient at the activation's output).
The same decision adds or removes dh[row, h] W1[e][h, :] from dx of the row's token.  The dW1
and dx checks therefore accept every combination of decisions at the pairs with an oracle
|z| < RELU_DELTA (about 1000x the GPU's accumulation error): each element must lie within
the tolerance plus the sum of |dh| |x| (dW1) or |dh| |W1| (dx) over its ambiguous pairs.  No
element is left out of the comparison.
"""
import numpy as np

RELU_DELTA = 1e-4


def relu_slacks(cfg, inp, r, dy):
    """Elementwise bounds on how far any choice of the ambiguous ReLU decisions moves dW1
    [E + Es, H, M] and dx [N, M], and the number of ambiguous (row, hidden unit) pairs.  Zero
    for other activations."""
    E, Es = cfg["n_experts"], cfg["n_shared"]
    slack = np.zeros(np.shape(inp.W1))
    slack_dx = np.zeros(np.shape(inp.x))
    if cfg["act"] != 0:
        return slack, slack_dx, 0
    x = np.asarray(inp.x, np.float64)
    dy = np.asarray(dy, np.float64)
    kept = r["pos"] >= 0
    n_amb = 0

    def add(e, rows, do):
        nonlocal n_amb
        w1 = np.asarray(inp.W1[e], np.float64)
        z = x[rows] @ w1.T
        amb = np.abs(z) < RELU_DELTA
        n_amb += int(amb.sum())
        if amb.any():
            a = np.abs(do @ np.asarray(inp.W2[e], np.float64)) * amb
            slack[e] += a.T @ np.abs(x[rows])
            slack_dx[rows] += a @ np.abs(w1)   # rows are distinct tokens

    for e in range(E):
        for j in range(cfg["top_k"]):
            rows = np.nonzero(kept[:, j] & (r["topk_idx"][:, j] == e))[0]
            if rows.size:
                add(e, rows, r["topk_w"][rows, j][:, None] * dy[rows])
    for q in range(Es):
        add(E + q, np.arange(cfg["n_tokens"]), dy)
    return slack, slack_dx, n_amb

