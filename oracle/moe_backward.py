"""Plain CPU oracle of the MoE layer's backward pass (float64).

TEST INFRASTRUCTURE ONLY, under the same rule as moe_oracle.py: only ``tests/``,
``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may use it, and it
shares no code with the HIP path.

The loss whose gradient is taken is

    L = sum_n <dy_n, y_n> + a_aux * aux + a_z * z_loss + a_dev * dev_loss,

so ``dy`` is the upstream gradient of the layer output and the three coefficients weight
the auxiliary losses ([GShard] "Top-2 gating 的四个机制 / Auxiliary loss": the aux loss is
added to the model loss with a coefficient; [MegaBlocks] "3. 负载均衡损失": the gradient of
the balance loss reaches the router only through the scores, the token counts being
constants; [Lec16] "MoE 训练中的负载均衡").  Routing decisions (top-k selection, group
limits, random routing, capacity drops) are piecewise constant and carry no gradient; every
other step is differentiated by the chain rule, written out here step by step:

  y_n    = [res] x_n + sum_j w_nj o_nj + sum_q SharedFFN_q(x_n),   w_nj = kept_nj * wpre_nj
  o      = act(x W1_e^T) W2_e^T        (gated: (Swish(x G^T) * (x U^T)) W2_e^T)
  wpre   = gate normalisation of the selected softmax probabilities p = softmax(l)
  l      = x Wg^T + bg

Results: dx [N, M], dWg [E, M], dbg [E], dW1 and dW2 (the shapes of W1 and W2), plus the
intermediate dlogits [N, E] and dw [N, k] (gradient of the kept combine weights).

Pinned in tests/test_backward_pins.py against central finite differences of the forward
oracle (float64 routing), on small layers that exercise every flag.
"""
import numpy as np
from scipy.special import erf as _erf

from oracle import moe_oracle as mo


def act_grad(z, act):
    """d act / dz for ReLU (act 0; 0 at z = 0) and exact GELU (act 1):
    GELU'(z) = Phi(z) + z phi(z), Phi the normal CDF, phi its density."""
    z = np.asarray(z, dtype=np.float64)
    if act == 0:
        return (z > 0).astype(np.float64)
    phi = np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)
    return 0.5 * (1.0 + _erf(z / np.sqrt(2.0))) + z * phi


def swish_grad(z):
    """d/dz z sigmoid(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))."""
    z = np.asarray(z, dtype=np.float64)
    sig = mo.swish(z) / np.where(z == 0, 1.0, z)
    sig = np.where(z == 0, 0.5, sig)
    return sig * (1.0 + z * (1.0 - sig))


def expert_backward(xrows, W1e, W2e, act, do):
    """One expert on a batch of rows: returns (dx rows, dW1e, dW2e, o) for upstream do.

    Forward: z = x W1e^T, h = act(z) (gated: h = Swish(g) * u with g, u the two halves of
    z), o = h W2e^T.  Backward: dh = do W2e, dW2e = do^T h, dz = dh * act'(z) (gated:
    dg = dh * u * Swish'(g), du = dh * Swish(g)), dW1e = dz^T x, dx = dz W1e.
    """
    x = np.asarray(xrows, np.float64)
    W1e = np.asarray(W1e, np.float64)
    W2e = np.asarray(W2e, np.float64)
    z = x @ W1e.T
    if act == mo.ACT_SWIGLU:
        H = W1e.shape[0] // 2
        g, u = z[:, :H], z[:, H:]
        h = mo.swish(g) * u
    else:
        h = mo.activation(z, act)
    o = h @ W2e.T
    dh = do @ W2e
    dW2e = do.T @ h
    if act == mo.ACT_SWIGLU:
        dz = np.concatenate([dh * u * swish_grad(g), dh * mo.swish(g)], axis=1)
    else:
        dz = dh * act_grad(z, act)
    dW1e = dz.T @ x
    dxr = dz @ W1e
    return dxr, dW1e, dW2e, o


def gate_weight_grad(p, idx, gate_norm, norm_p, dw):
    """dL/dp [N, E] from dL/dwpre [N, k] through the gate normalisation (R-norm, R-pnorm).

    none: wpre_j = p_j.  p-norm (sum is P = 1): wpre_j = p_j / D, D = (sum_i p_i^P)^(1/P)
    over the selected experts, so dwpre_j/dp_i = [i = j] / D - p_j p_i^(P-1) D^(-1-P), and
    dL/dp_i = dw_i / D - p_i^(P-1) D^(-1-P) sum_j dw_j p_j (unselected experts get 0).
    """
    N, E = p.shape
    dp = np.zeros((N, E))
    ps = np.take_along_axis(p, idx.astype(np.int64), axis=1)       # [N, k]
    if gate_norm == 0:
        dps = dw
    else:
        P = 1.0 if gate_norm == 1 else float(norm_p)
        D = (ps ** P).sum(axis=1, keepdims=True) ** (1.0 / P)
        s = (dw * ps).sum(axis=1, keepdims=True)
        dps = dw / D - ps ** (P - 1.0) * D ** (-1.0 - P) * s
    for j in range(idx.shape[1]):
        dp[np.arange(N), idx[:, j]] += dps[:, j]
    return dp


def balance_grad(cfg, idx, coef_aux, coef_dev):
    """dL/dp [N, E] of a_aux * aux + a_dev * dev_loss; the selection counts c are constants.

    Per token group g of S tokens: aux = (1/G) E/(k S) sum_e m_e c_e with m_e = (1/S) sum_n
    p_ne gives a_aux E c_ge / (G k S^2); dev = (1/G) sum_j f_j P_j with f_j the mean of
    f_e = E c_e / (k S) over expert group j and P_j = sum_{e in j} m_e gives
    a_dev f_j(e) / (G S).
    """
    N, k = idx.shape
    E, G = cfg["n_experts"], cfg["n_groups"]
    D = cfg.get("expert_groups", 1)
    dp = np.zeros((N, E))
    if N == 0:
        return dp
    S = N // G
    gs = E // D
    cnt = np.zeros((G, E))
    for n in range(N):
        for j in range(k):
            cnt[n // S, idx[n, j]] += 1.0
    for g in range(G):
        rows = slice(g * S, (g + 1) * S)
        dp[rows] += coef_aux * E * cnt[g][None, :] / (G * k * S * S)
        f = E * cnt[g] / (k * S)
        fj = f.reshape(D, gs).mean(axis=1)
        dp[rows] += coef_dev * np.repeat(fj, gs)[None, :] / (G * S)
    return dp


def softmax_grad(p, dp):
    """Softmax backward: dL/dl_e = p_e (dL/dp_e - sum_i p_i dL/dp_i)."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def z_loss_grad(l, p, coef_z):
    """d(a_z z_loss)/dl: z = (1/N) sum_n lse_n^2 and d lse_n / d l_ne = p_ne."""
    N = l.shape[0]
    if N == 0:
        return np.zeros_like(p)
    mx = l.max(axis=1, keepdims=True)
    lse = mx + np.log(np.exp(l - mx).sum(axis=1, keepdims=True))
    return coef_z * 2.0 * lse * p / N


def router_backward(cfg, p, idx, lr, dw, coef_aux=0.0, coef_z=0.0, coef_dev=0.0):
    """dL/dl [N, E] from the combine weights' gradient dw [N, k]: through the gate weights
    (gate_weight_grad), plus the balance losses, then the softmax, plus the z-loss.  p: the
    softmax probabilities, idx: the selection, lr: the logits (float64)."""
    dp = gate_weight_grad(p, idx, cfg["gate_norm"], cfg.get("norm_p", 1.0), dw)
    dp += balance_grad(cfg, idx, coef_aux, coef_dev)
    return softmax_grad(p, dp) + z_loss_grad(lr, p, coef_z)


def layer_backward(cfg, x, Wg, bg, W1, W2, u, dy, coef_aux=0.0, coef_z=0.0, coef_dev=0.0,
                   logits=None, exact=False):
    """Gradients of L (module docstring) with respect to x, Wg, bg, W1, W2.

    ``logits``: the routing logits to use (the same-logits protocol with the GPU); by
    default this oracle's own, rounded to fp32 unless ``exact``.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    N, M = x.shape
    E, Es, k = cfg["n_experts"], cfg["n_shared"], cfg["top_k"]
    G = cfg["n_groups"]
    act = cfg["act"]
    if logits is None:
        logits = mo.router_logits(x, Wg, bg)
        if not exact:
            logits = logits.astype(np.float32)
    r = mo.route(cfg, logits, u, exact=exact)
    lr = np.asarray(logits, np.float64 if exact else np.float32).astype(np.float64)
    p = r["p"]
    idx, pos, wk = r["topk_idx"], r["pos"], r["topk_w"]
    kept = pos >= 0

    dx = dy.copy() if cfg["residual"] else np.zeros_like(x)
    dW1 = np.zeros(np.shape(W1))
    dW2 = np.zeros(np.shape(W2))
    dw = np.zeros((N, k))
    # routed experts: rows that chose expert e at rank j (kept slots only)
    for e in range(E):
        for j in range(k):
            sel = np.nonzero(kept[:, j] & (idx[:, j] == e))[0]
            if sel.size == 0:
                continue
            do = wk[sel, j][:, None] * dy[sel]
            dxr, dW1e, dW2e, o = expert_backward(x[sel], W1[e], W2[e], act, do)
            dx[sel] += dxr
            dW1[e] += dW1e
            dW2[e] += dW2e
            dw[sel, j] = (dy[sel] * o).sum(axis=1)
    # shared experts: weight 1, every token
    for q in range(Es):
        dxr, dW1e, dW2e, _ = expert_backward(x, W1[E + q], W2[E + q], act, dy)
        dx += dxr
        dW1[E + q] += dW1e
        dW2[E + q] += dW2e

    dl = router_backward(cfg, p, idx, lr, dw, coef_aux, coef_z, coef_dev)
    dWg = dl.T @ x
    dbg = dl.sum(axis=0)
    dx += dl @ np.asarray(Wg, np.float64)
    return dict(dx=dx, dWg=dWg, dbg=dbg, dW1=dW1, dW2=dW2, dlogits=dl, dw=dw, routing=r)


def loss(cfg, x, Wg, bg, W1, W2, u, dy, coef_aux=0.0, coef_z=0.0, coef_dev=0.0):
    """The scalar L of the module docstring from the forward oracle, float64 routing."""
    logits = mo.router_logits(x, Wg, bg)
    r = mo.route(cfg, logits, u, exact=True)
    y = mo.layer_outputs(cfg, x, W1, W2, r)
    return (float((np.asarray(dy, np.float64) * y).sum()) + coef_aux * r["aux"] +
            coef_z * r["z_loss"] + coef_dev * r["dev_loss"]), r
