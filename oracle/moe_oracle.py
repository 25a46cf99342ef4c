"""Plain, slow CPU oracle for the single-GPU MoE layer forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It imports nothing
from the HIP product path and the product path never imports it; the two share no code.
All floating point runs in float64 on the exact values of the (fp32 or bf16) inputs.

Sources, cited by page title and section:
  [GShard]     "GShard: Scaling Giant Models with Conditional Computation and Automatic
               Sharding" -- reading notes (process-cxr.github.io).
  [MegaBlocks] "04 · 路由、负载均衡与专家并行" -- MegaBlocks router / parallelism chapter
               (ai-reference-codex.pages.dev).
  [Lec16]      "Lec16 Systems for MoE Models" -- CMU 11-868 lecture notes (xloverflow.github.io).
  [11-868 #12] CMU 11-868 LLM Systems reading #12, model and expert parallelism
               (quidproquo.cc).

Where the pages are silent, garbled or disagree, the reading taken is stated at the
function that depends on it, and summarised here:
  R-norm   top-k selection is made on the logits (softmax is monotone, so this is the
           same set as selecting on the softmax); norm=sum gives w_j = p_j / sum_sel p
           (the "softmax over the selected logits" of [Lec16] and the renormalised top-k
           of [MegaBlocks]); norm=none gives w_j = p_j (the Switch top-1 gate, [Lec16]).
  R-tie    ties between equal logits go to the lower expert index.
  R-order  capacity positions are assigned rank-major: every token's 1st choice in
           token order, then every 2nd choice, and so on.
  R-part   a slot that finds its expert full is lost on its own; a token is dropped
           (residual only) when all of its slots are lost.
  R-rr     the 2nd expert is kept with probability 2*w2, w2 = p2/(p1+p2), decided as
           u < 2*w2 in float64 from the two fp32 logits; a skipped slot takes no
           capacity and gets weight 0.
  R-aux    aux = mean over groups of E * sum_e m_e * c_e / (k*S), c_e counting the top-k
           selections before capacity and random routing.
  R-res    the layer output includes the residual: y = x + sum_j w_j FFN_e_j(x) (+ shared
           experts); a fully dropped token gets y = x.  residual=0 gives the bare layer.
  R-ffn    expert = act(x W1^T) W2^T, no biases; GELU is the exact erf form.
  R-glu    the gated expert of [Lec16] "DeepSeek V3 MoE (670B)", (Swish(x W1) * (x W2)) W3,
           takes Swish with beta = 1 (z * sigmoid(z), also called SiLU).  Its two input
           projections are stacked in one weight: W1[e] is [2H, M], rows 0..H-1 the
           Swish (gate) projection and rows H..2H-1 the linear (up) one; W2[e] [M, H]
           holds the output projection (the formula's W3).
  R-empty  an empty batch (N = 0) routes nothing and has aux = 0 (and z-loss 0).
  R-pnorm  the optional p-norm renormalisation of [MegaBlocks] section 2 divides the k
           selected probabilities by their p-norm, (sum_i p_i^P)^(1/P), P > 0 a real
           number (P = 1 is the sum normalisation); gate_norm == 2 selects it.
  R-grp    group-limited routing ([Lec16] "DeepSeek V3 MoE (670B)": 8 expert groups, 4
           "limited groups"): the E experts form D contiguous groups of E/D; a group's score
           is the largest logit among its experts (equivalently its largest softmax score);
           each token keeps the topk_groups best groups (ties to the lower group index)
           and picks its top-k experts among theirs only.  D = 1 is plain top-k.
  R-dev    the device-level balance loss of [Lec16] "DeepSeek MoE 的负载均衡" groups the
           expert-level terms by the same D groups: per token group, sum_j f_j P_j with
           f_j the mean over group j of f_i = E c_i / (k S) and P_j the sum over group j of
           P_i = m_i; averaged over token groups like the aux loss.
  R-z      the router z-loss of [MegaBlocks] section 2 is the mean over all N tokens of
           logsumexp(logits_n)^2, on the fp32 logits that feed the softmax (router offsets
           included), one number per layer whatever the grouping.

Pins: every public function here is checked by ``tests/test_oracle_pins.py`` against
closed forms, invariants, the dense one-hot formulation in ``einsum_oracle.py``, brute
force on tiny inputs, the worked dispatch example of [MegaBlocks] (tests/golden/) and
special cases that reduce to a library matmul.  The readings above are choices among
the pages' descriptions; their fidelity to the original systems is parity unpinned.
"""
import numpy as np
from scipy.special import erf as _erf


# --------------------------------------------------------------------------- router

def router_logits(x, Wg, bg=None):
    """logits[n, e] = sum_m x[n, m] * Wg[e, m] (+ bg[e]), in float64.

    [MegaBlocks] "2. 路由器：一个线性层的全部戏份": the router is one bias-free linear
    layer from the hidden size to E.  Wg is stored [E, M] (row e = expert e's gate
    vector).  The optional bg adds a fixed per-expert offset (the skewed-router inputs).
    """
    x = np.asarray(x, dtype=np.float64)
    Wg = np.asarray(Wg, dtype=np.float64)
    logits = x @ Wg.T
    if bg is not None:
        logits = logits + np.asarray(bg, dtype=np.float64)[None, :]
    return logits


def softmax(logits):
    """Row softmax over all E experts, float64, max-subtracted.

    [Lec16] "Switch Transformer": G(x) = Softmax(x W_g); [MegaBlocks] section 2 keeps
    the full-E scores for the load-balancing loss.
    """
    l = np.asarray(logits, dtype=np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def topk_experts(logits, k):
    """Indices of the k largest logits per token, in descending order (R-tie).

    [Lec16] "Switch Transformer" (KeepTopK); [MegaBlocks] section 2 (softmax -> top-k).
    A stable sort of the negated logits puts equal logits in ascending expert order.
    """
    l = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-l, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def expert_group_mask(logits, n_expert_groups, topk_groups):
    """Experts each token may route to under group-limited routing (R-grp), bool [N, E].

    Group d holds experts [d E/D, (d+1) E/D).  Its score is the largest logit of its
    experts; the topk_groups best groups of a token (stable order: ties to the lower group
    index) are allowed.  With D == 1 every expert is allowed.
    """
    l = np.asarray(logits, dtype=np.float64)
    N, E = l.shape
    D = int(n_expert_groups)
    allowed = np.ones((N, E), dtype=bool)
    if D <= 1:
        return allowed
    gs = E // D
    for n in range(N):
        score = np.array([l[n, d * gs:(d + 1) * gs].max() for d in range(D)])
        keep = np.argsort(-score, kind="stable")[:topk_groups]
        allowed[n] = False
        for d in keep:
            allowed[n, d * gs:(d + 1) * gs] = True
    return allowed


def gate_weights(p, idx, gate_norm, norm_p=1.0):
    """Pre-drop combine weights of the selected experts (R-norm, R-pnorm).

    gate_norm == 1: w_j = p_j / sum_i p_i over the k selected experts -- equal to a
    softmax over the selected logits ([Lec16] "Switch Transformer", "共享专家 vs. 路由专家")
    and to the renormalised top-k of [MegaBlocks] section 2.  gate_norm == 0: w_j = p_j.
    gate_norm == 2: w_j = p_j / (sum_i p_i^P)^(1/P), the p-norm option of [MegaBlocks]
    section 2 ("权重归一化"), P = norm_p.
    """
    psel = np.take_along_axis(np.asarray(p, dtype=np.float64), idx.astype(np.int64), axis=1)
    if gate_norm == 1:
        return psel / psel.sum(axis=1, keepdims=True)
    if gate_norm == 2:
        P = float(norm_p)
        return psel / ((psel ** P).sum(axis=1, keepdims=True) ** (1.0 / P))
    return psel


def z_loss(logits32):
    """Router z-loss (R-z): mean_n (log sum_e exp(l_{n,e}))^2, float64.

    [MegaBlocks] section 2 ("z-loss ... mean(logsumexp(logits)²)"): it penalises large
    router logits.  logsumexp is evaluated max-shifted.  An empty batch gives 0.
    """
    l = np.asarray(logits32, dtype=np.float64)
    if l.shape[0] == 0:
        return 0.0
    mx = l.max(axis=1)
    lse = mx + np.log(np.exp(l - mx[:, None]).sum(axis=1))
    return float(np.mean(lse * lse))


def random_routing_keep(logits32, idx, u):
    """Whether each token's 2nd-choice slot is dispatched (R-rr), k == 2 only.

    [GShard] "Top-2 gating 的四个机制 / Random routing": the 2nd expert is used with a
    probability proportional to its gate.  With w2 = p2/(p1+p2) = 1/(1+exp(l1-l2)) the
    slot is kept iff u < 2*w2, evaluated in float64 from the fp32 logits l1 >= l2.
    Returns a bool array [N].
    """
    l = np.asarray(logits32, dtype=np.float32).astype(np.float64)
    n = np.arange(l.shape[0])
    l1 = l[n, idx[:, 0]]
    l2 = l[n, idx[:, 1]]
    threshold = 2.0 / (1.0 + np.exp(l1 - l2))
    return np.asarray(u, dtype=np.float32).astype(np.float64) < threshold


# --------------------------------------------------------------------------- capacity

def assign_positions(idx, active, n_groups, n_experts, capacity):
    """Capacity positions by the sequential counter of the definition (R-order, R-part).

    [GShard] "Top-2 gating 的四个机制 / Expert capacity" and "Local group dispatching":
    the batch is split into G equal groups that route independently, each expert takes
    at most C tokens per group, and a slot beyond capacity is not computed.

    For each group, counters start at 0; ranks are visited in order and, within a rank,
    tokens in ascending order.  An active slot whose expert's counter is below C takes
    the counter's value as its position and bumps the counter; otherwise it is dropped.
    Inactive slots take nothing.  Returns pos [N, k] (-1 = not kept) and count [G, E].
    """
    N, k = idx.shape
    G = n_groups
    S = N // G if G else 0
    pos = np.full((N, k), -1, dtype=np.int32)
    count = np.zeros((G, n_experts), dtype=np.int32)
    for g in range(G):
        cnt = [0] * n_experts
        for j in range(k):
            for n in range(g * S, (g + 1) * S):
                if not active[n, j]:
                    continue
                e = int(idx[n, j])
                if cnt[e] < capacity:
                    pos[n, j] = cnt[e]
                    cnt[e] += 1
        count[g, :] = cnt
    return pos, count


def dispatch_rows(idx, pos, count):
    """Rows of the compact expert-major buffer, ordered (expert, group, position).

    [GShard] "Sharding 与 MoE 的交替布局": the group-major tokens are regrouped into an
    expert-major buffer; here the unused capacity is squeezed out, so expert e's rows
    start at offset[e] = sum_{e'<e} sum_g count[g, e'] and group g's block inside it
    starts after the earlier groups' counts.  Returns offset [E+1] and row [N, k]
    (-1 where the slot is not kept).
    """
    G, E = count.shape
    N, k = idx.shape
    S = N // G if G else 0
    totals = count.sum(axis=0)
    offset = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offset[e + 1] = offset[e] + totals[e]
    row = np.full((N, k), -1, dtype=np.int32)
    for n in range(N):
        g = n // S
        for j in range(k):
            if pos[n, j] >= 0:
                e = int(idx[n, j])
                row[n, j] = offset[e] + count[:g, e].sum() + pos[n, j]
    return offset.astype(np.int32), row


def aux_loss(p, idx, n_groups, n_experts):
    """Auxiliary load-balancing loss (R-aux).

    [GShard] "Top-2 gating 的四个机制 / Auxiliary loss" defines c_e/S (the share of the
    group's tokens sent to expert e) and m_e (the expert's mean gate) and uses m_e*c_e/S
    as the differentiable proxy; [MegaBlocks] "3. 负载均衡损失" scales the dot product of
    tokens-per-expert and mean scores by E/(T*k); [Lec16] "DeepSeek MoE 的负载均衡" uses
    f_i = (E/k) * count_i / T.  Per group: E * sum_e m_e * c_e / (k*S); averaged over groups.
    """
    N, k = idx.shape
    G = n_groups
    if N == 0:
        return 0.0
    S = N // G
    total = 0.0
    for g in range(G):
        pg = np.asarray(p[g * S:(g + 1) * S], dtype=np.float64)
        m = pg.sum(axis=0) / S
        c = np.zeros(n_experts, dtype=np.float64)
        for n in range(g * S, (g + 1) * S):
            for j in range(k):
                c[idx[n, j]] += 1.0
        total += n_experts * float(np.dot(m, c)) / (k * S)
    return total / G


def dev_loss(p, idx, n_groups, n_experts, n_expert_groups):
    """Device-level balance loss (R-dev), the expert-level terms summed per expert group.

    [Lec16] "DeepSeek MoE 的负载均衡": L_DevBal = sum_j f_j P_j with f_j the mean f of the
    experts in group j and P_j the sum of their P; f_i = (E/k) * (tokens to i) / T and
    P_i = mean routing score, as in the expert-level loss (computed per token group of S
    tokens, then averaged over the G token groups).  An empty batch gives 0.
    """
    N, k = idx.shape
    G, E, D = n_groups, n_experts, int(n_expert_groups)
    if N == 0:
        return 0.0
    S = N // G
    gs = E // D
    total = 0.0
    for g in range(G):
        P = np.asarray(p[g * S:(g + 1) * S], dtype=np.float64).sum(axis=0) / S
        cnt = np.zeros(E, dtype=np.float64)
        for n in range(g * S, (g + 1) * S):
            for j in range(k):
                cnt[idx[n, j]] += 1.0
        f = E * cnt / (k * S)
        for d in range(D):
            total += f[d * gs:(d + 1) * gs].mean() * P[d * gs:(d + 1) * gs].sum()
    return total / G


def route(cfg, logits32, u=None, exact=False):
    """Routing, positions, dispatch rows and aux from given fp32 logits (no FFN).

    Mirrors the C ABI's ``moe_route``: the same steps the layer runs after the router
    GEMM.  ``logits32`` is treated as exact fp32 values; with ``exact=True`` float64 logits
    are used as given (no rounding), for finite-difference checks of the backward pass.
    """
    N, E, k = cfg["n_tokens"], cfg["n_experts"], cfg["top_k"]
    G, C = cfg["n_groups"], cfg["capacity"]
    l32 = np.asarray(logits32, dtype=np.float64 if exact else np.float32).reshape(N, E)
    if N == 0:
        z = np.zeros((0, k), dtype=np.int32)
        return dict(topk_idx=z, active=z.astype(bool), pos=z, row=z,
                    topk_w=np.zeros((0, k)), w_pre=np.zeros((0, k)),
                    count=np.zeros((G, E), np.int32), offset=np.zeros(E + 1, np.int32),
                    aux=0.0, z_loss=0.0, dev_loss=0.0, stats=np.zeros(4, np.int64),
                    p=np.zeros((0, E)))
    p = softmax(l32)
    D, TG = cfg.get("expert_groups", 1), cfg.get("topk_groups", 1)
    allowed = expert_group_mask(l32, D, TG)
    idx = topk_experts(np.where(allowed, l32.astype(np.float64), -np.inf), k)
    w_pre = gate_weights(p, idx, cfg["gate_norm"], cfg.get("norm_p", 1.0))
    active = np.ones((N, k), dtype=bool)
    if cfg["random_routing"]:
        if k != 2 or u is None:
            raise ValueError("random routing needs top_k == 2 and u")
        active[:, 1] = random_routing_keep(l32, idx, u)
    pos, count = assign_positions(idx, active, G, E, C)
    kept = pos >= 0
    offset, row = dispatch_rows(idx, pos, count)
    topk_w = np.where(kept, w_pre, 0.0)          # no renormalisation after drops
    aux = aux_loss(p, idx, G, E)
    n_active = int(active.sum())
    R = int(kept.sum())
    stats = np.array([R, n_active - R, int((~kept.any(axis=1)).sum()), N * k - n_active],
                     dtype=np.int64)
    return dict(topk_idx=idx, active=active, pos=pos, row=row, topk_w=topk_w,
                w_pre=w_pre, count=count, offset=offset, aux=aux, z_loss=z_loss(l32),
                dev_loss=dev_loss(p, idx, G, E, D), stats=stats, p=p)


# --------------------------------------------------------------------------- experts

ACT_SWIGLU = 2


def activation(z, act):
    """ReLU (act 0) or exact GELU (act 1): 0.5 z (1 + erf(z / sqrt 2)) (R-ffn)."""
    z = np.asarray(z, dtype=np.float64)
    if act == 0:
        return np.maximum(z, 0.0)
    if act == 1:
        return 0.5 * z * (1.0 + _erf(z / np.sqrt(2.0)))
    raise ValueError("the gated expert's activation acts on two projections (expert_ffn)")


def swish(z):
    """Swish with beta = 1: z * sigmoid(z), float64 (R-glu).

    sigmoid(z) = 1 / (1 + exp(-z)) is evaluated from exp(-|z|), which never overflows.
    """
    z = np.asarray(z, dtype=np.float64)
    t = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + t), t / (1.0 + t))
    return z * sig


def expert_ffn(xrows, W1e, W2e, act):
    """One expert on a batch of token rows, float64, no biases.

    act 0/1: act(x W1e^T) W2e^T.  [GShard] "MoE Transformer": each expert is a two-layer
    network of the dense FFN's shape; W1e is [H, M] (row n feeds hidden unit n), W2e is
    [M, H].
    act 2 (gated): (Swish(x G^T) * (x U^T)) W2e^T with G = W1e[:H], U = W1e[H:] (R-glu);
    [Lec16] "DeepSeek V3 MoE (670B)": every expert uses this SwiGLU form.
    """
    x = np.asarray(xrows, np.float64)
    W1e = np.asarray(W1e, np.float64)
    if act == ACT_SWIGLU:
        H = W1e.shape[0] // 2
        h = swish(x @ W1e[:H].T) * (x @ W1e[H:].T)
    else:
        h = activation(x @ W1e.T, act)
    return h @ np.asarray(W2e, np.float64).T


def layer_outputs(cfg, x, W1, W2, routing, tokens=None):
    """y for the given tokens (all if None), float64, from a routing dict (R-res).

    y_n = [residual] x_n + sum_j w_{n,j} FFN_{e_{n,j}}(x_n) + sum_q SharedFFN_q(x_n).
    [GShard] "MoE Transformer" (gate-weighted sum of at most two experts) and
    "Capacity overflow 会跳过 expert computation" (a dropped token passes through the
    residual); [Lec16] "共享专家 vs. 路由专家" (shared experts are always on and add
    with weight 1).  Experts are evaluated in batches of the rows that chose them.
    """
    N, M = x.shape
    E, Es, k = cfg["n_experts"], cfg["n_shared"], cfg["top_k"]
    toks = np.arange(N) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xs = np.asarray(x[toks], dtype=np.float64)
    y = xs.copy() if cfg["residual"] else np.zeros_like(xs)
    idx = routing["topk_idx"][toks]
    kept = routing["pos"][toks] >= 0
    w = routing["topk_w"][toks]
    routed = np.zeros_like(xs)
    for e in range(E):
        for j in range(k):
            sel = np.nonzero(kept[:, j] & (idx[:, j] == e))[0]
            if sel.size == 0:
                continue
            out = expert_ffn(xs[sel], W1[e], W2[e], cfg["act"])
            routed[sel] += w[sel, j][:, None] * out
    shared = np.zeros_like(xs)
    for q in range(Es):
        shared += expert_ffn(xs, W1[E + q], W2[E + q], cfg["act"])
    return y + routed + shared


def moe_forward(cfg, inp, tokens=None, logits32=None):
    """Whole layer: logits (float64, stored fp32 for routing), routing, outputs, aux.

    ``inp`` is a synth.Inputs-like object with x, Wg, W1, W2 (fp32 arrays of exact
    values), bg and u.  If ``logits32`` is given, routing runs on those logits (the
    same-logits protocol); otherwise on this oracle's own logits rounded to fp32.
    """
    logits = router_logits(inp.x, inp.Wg, inp.bg)
    l32 = logits.astype(np.float32) if logits32 is None else np.asarray(logits32, np.float32)
    r = route(cfg, l32, inp.u)
    r["logits"] = logits
    r["y"] = layer_outputs(cfg, inp.x, inp.W1, inp.W2, r, tokens)
    return r
