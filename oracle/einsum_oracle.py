"""Second, independent CPU formulation of the MoE layer: dense one-hot masks + einsum.

TEST INFRASTRUCTURE ONLY (same rule as moe_oracle.py: only tests/, smoke() and the
benchmark's cpu_baseline leg may use it).  It shares no code with moe_oracle.py.

[GShard] "Automatic propagation 与 manual override" states that dispatch can be written
as a one-hot einsum or as an index tensor plus a local Gather.  moe_oracle.py is the
index/counter form; this is the one-hot form: per group, dispatch and combine tensors of
shape [S, E, C] are built from cumulative sums of one-hot expert masks, the tokens are
dispatched with an einsum into a padded [E, G, C, M] buffer, every expert runs on its
[G*C, M] slice (padding included; padded rows never reach the output because their
combine weight is zero, [GShard] "Static shape 与 uneven partition"), and the outputs
are combined with a second einsum.  Float64 throughout, small inputs only.
"""
import numpy as np
from scipy.special import erf, expit, logsumexp


def _hidden(rows, W1e, act):
    """Hidden layer of one expert.  The gated form (act 2, [Lec16] "DeepSeek V3 MoE
    (670B)") multiplies z*sigmoid(z) of the first H projections by the last H ones;
    the sigmoid is scipy's expit."""
    pre = rows @ np.asarray(W1e, np.float64).T
    if act == 0:
        return np.maximum(pre, 0.0)
    if act == 1:
        return 0.5 * pre * (1.0 + erf(pre / np.sqrt(2.0)))
    H = pre.shape[1] // 2
    g, up = pre[:, :H], pre[:, H:]
    return g * expit(g) * up


def einsum_layer(cfg, x, Wg, W1, W2, bg=None, u=None, logits32=None):
    N, M = x.shape
    E, Es, k = cfg["n_experts"], cfg["n_shared"], cfg["top_k"]
    G, C = cfg["n_groups"], cfg["capacity"]
    S = N // G
    x = np.asarray(x, np.float64)
    if logits32 is None:
        lg = np.einsum("nm,em->ne", x, np.asarray(Wg, np.float64))
        if bg is not None:
            lg = lg + np.asarray(bg, np.float64)
        lg = lg.astype(np.float32)
    lg = np.asarray(logits32 if logits32 is not None else lg, np.float32).astype(np.float64)

    # Gates: full softmax, then successive argmax with lower index winning ties.
    ex = np.exp(lg - lg.max(axis=1, keepdims=True))
    probs = ex / ex.sum(axis=1, keepdims=True)
    D, TG = cfg.get("expert_groups", 1), cfg.get("topk_groups", 1)
    remaining = lg.copy()
    if D > 1:
        # group-limited routing: a group's rank counts the groups with a larger best logit
        # (and the lower-indexed ones with an equal one); ranks below TG are allowed
        gmax = lg.reshape(N, D, E // D).max(axis=2)                       # [N, D]
        gt = (gmax[:, None, :] > gmax[:, :, None]).sum(axis=2)
        eq_before = ((gmax[:, None, :] == gmax[:, :, None]) &
                     (np.arange(D)[None, None, :] < np.arange(D)[None, :, None])).sum(axis=2)
        ok = np.repeat((gt + eq_before) < TG, E // D, axis=1)             # [N, E]
        remaining = np.where(ok, remaining, -np.inf)
    onehots, psel = [], []
    for _ in range(k):
        best = remaining.argmax(axis=1)           # first maximum = lowest index
        oh = np.eye(E)[best]                       # [N, E]
        onehots.append(oh)
        psel.append((probs * oh).sum(axis=1))
        remaining = np.where(oh > 0, -np.inf, remaining)
    psel = np.stack(psel, axis=1)                  # [N, k]
    sel = sum(onehots)                             # [N, E] top-k selections (pre-capacity)
    if cfg["gate_norm"] == 2:                      # p-norm of the selected probabilities
        P = float(cfg.get("norm_p", 1.0))
        w = psel / np.linalg.norm(psel, ord=P, axis=1, keepdims=True) if P >= 1 else \
            psel / (psel ** P).sum(axis=1, keepdims=True) ** (1.0 / P)
    else:
        w = psel / psel.sum(axis=1, keepdims=True) if cfg["gate_norm"] else psel

    if cfg["random_routing"]:
        l1 = (lg * onehots[0]).sum(axis=1)
        l2 = (lg * onehots[1]).sum(axis=1)
        keep2 = np.asarray(u, np.float32).astype(np.float64) < 2.0 / (1.0 + np.exp(l1 - l2))
        onehots[1] = onehots[1] * keep2[:, None]

    # Capacity by cumulative sums inside each group, rank by rank.
    dispatch = np.zeros((G, S, E, C))
    combine = np.zeros((G, S, E, C))
    for g in range(G):
        used = np.zeros(E)                         # slots already filled per expert
        for j in range(k):
            mask = onehots[j][g * S:(g + 1) * S]   # [S, E]
            loc = np.cumsum(mask, axis=0) - 1 + used[None, :]
            mask = mask * (loc < C)
            used = used + mask.sum(axis=0)
            loc_tok = (loc * mask).sum(axis=1).astype(np.int64)   # [S]
            slot = np.eye(C)[np.clip(loc_tok, 0, C - 1)]            # [S, C]
            d = mask[:, :, None] * slot[:, None, :]                 # [S, E, C]
            dispatch[g] += d
            combine[g] += d * w[g * S:(g + 1) * S, j][:, None, None]

    xg = x.reshape(G, S, M)
    buf = np.einsum("gsec,gsm->egcm", dispatch, xg)                 # [E, G, C, M]
    out = np.zeros_like(buf)
    for e in range(E):
        rows = buf[e].reshape(G * C, M)
        h = _hidden(rows, W1[e], cfg["act"])
        out[e] = (h @ np.asarray(W2[e], np.float64).T).reshape(G, C, M)
    y = np.einsum("gsec,egcm->gsm", combine, out).reshape(N, M)
    for q in range(Es):
        h = _hidden(x, W1[E + q], cfg["act"])
        y = y + h @ np.asarray(W2[E + q], np.float64).T
    if cfg["residual"]:
        y = y + x

    # Aux and device-level losses from the dense masks (pre-capacity selections).
    aux = dev = 0.0
    for g in range(G):
        m = probs[g * S:(g + 1) * S].mean(axis=0)
        c = sel[g * S:(g + 1) * S].sum(axis=0)
        aux += E * float((m * c).sum()) / (k * S)
        f = E * c / (k * S)
        dev += float((f.reshape(D, E // D).mean(axis=1) * m.reshape(D, E // D).sum(axis=1)).sum())
    aux /= G
    dev /= G
    counts = dispatch.sum(axis=(1, 3))            # [G, E]
    z = float(np.mean(logsumexp(lg, axis=1) ** 2)) if N else 0.0   # router z-loss
    return dict(y=y, aux=aux, z_loss=z, dev_loss=dev, dispatch=dispatch, combine=combine,
                count=counts.astype(np.int32), logits=lg)
