"""Shared helpers of the GPU tests: upload seeded inputs, run the HIP path through the C ABI,
and compare with the CPU oracle under the same-logits protocol.

Same-logits protocol: the oracle's routing steps run on the logits the GPU produced, so
routing, positions, rows, counts, offsets and stats must match bit for bit; the GPU logits
themselves are compared with the oracle's float64 x Wg^T within tolerance, and the layer
output y with the oracle's float64 output computed from the (shared) routing.
"""
import sys

import numpy as np

from mixture_experts_layer_group_amd import binding, synth
from oracle import moe_oracle as mo

# Tolerances: max|gpu - ref| / max|ref| (per the layer dtype), aux relative.
Y_TOL = {0: 1e-4, 1: 2e-2}
LOGIT_TOL = 1e-4
AUX_TOL = 1e-5
W_TOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(inp, cfg):
    import torch
    dev = "cuda"

    def t(name):
        bits = getattr(inp, name + "_bits")
        if bits is not None:
            return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(getattr(inp, name)).to(dev)
    d = {n: t(n) for n in ("x", "Wg", "W1", "W2")}
    d["bg"] = torch.from_numpy(inp.bg).to(dev) if inp.bg is not None else None
    d["u"] = torch.from_numpy(inp.u).to(dev) if inp.u is not None else None
    return d


def run_gpu(cfg, dev, workspace=None):
    import torch
    y, aux, meta = binding.forward(cfg, dev["x"], dev["Wg"], dev["W1"], dev["W2"],
                                   bg=dev["bg"], u=dev["u"], workspace=workspace)
    torch.cuda.synchronize()
    out = meta.to_numpy()
    out["y"] = y.float().cpu().numpy()
    out["aux"] = float(aux.cpu().numpy()[0])
    out["z_loss"] = float(out["z_loss"][0])
    out["dev_loss"] = float(out["dev_loss"][0])
    return out


def rr_margin(cfg, logits32, idx, u):
    """Smallest |u - t| / t over tokens, t = 2 / (1 + exp(l1 - l2)) (the RR threshold)."""
    if not cfg["random_routing"] or cfg["n_tokens"] == 0:
        return np.inf
    l = logits32.astype(np.float64)
    n = np.arange(l.shape[0])
    t = 2.0 / (1.0 + np.exp(l[n, idx[:, 0]] - l[n, idx[:, 1]]))
    return float(np.min(np.abs(u.astype(np.float64) - t) / t))


def check_routing(cfg, g, ref):
    """Bit-exact integer outputs, weights within W_TOL, aux and z-loss within AUX_TOL
    relative."""
    for f in ("topk_idx", "pos", "row", "count", "offset"):
        a, b = np.asarray(g[f]), np.asarray(ref[f]).astype(np.int64)
        assert a.shape == b.shape, (f, a.shape, b.shape)
        bad = np.nonzero(a.astype(np.int64) != b)
        assert bad[0].size == 0, f"{f} differs at {bad[0][:5]}: gpu {a[bad][:5]} ref {b[bad][:5]}"
    assert (np.asarray(g["stats"]).astype(np.int64) == ref["stats"]).all(), (g["stats"], ref["stats"])
    dw = np.abs(g["topk_w"].astype(np.float64) - ref["topk_w"]).max() if g["topk_w"].size else 0.0
    assert dw <= W_TOL, f"topk_w max abs diff {dw}"
    if ref["aux"] != 0:
        rel = abs(g["aux"] - ref["aux"]) / abs(ref["aux"])
        assert rel <= AUX_TOL, f"aux {g['aux']} vs {ref['aux']} (rel {rel})"
    else:
        assert g["aux"] == 0.0
    for f in ("z_loss", "dev_loss"):
        if f not in g:
            continue
        if ref[f] != 0:
            rel = abs(g[f] - ref[f]) / abs(ref[f])
            assert rel <= AUX_TOL, f"{f} {g[f]} vs {ref[f]} (rel {rel})"
        else:
            assert g[f] == 0.0


def rel_err(a, ref):
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(np.asarray(a, np.float64) - ref).max() / (den if den > 0 else 1.0))


def sample_tokens(cfg, ref, n_sample, seed=0):
    """Seeded sample + every fully dropped token + one kept row of each non-empty expert."""
    N = cfg["n_tokens"]
    if n_sample is None or n_sample >= N:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    s = set(rng.choice(N, size=n_sample, replace=False).tolist())
    kept = ref["pos"] >= 0
    s.update(np.nonzero(~kept.any(axis=1))[0].tolist())
    for e in range(cfg["n_experts"]):
        hit = np.nonzero((ref["topk_idx"] == e) & kept)[0]
        if hit.size:
            s.add(int(hit[0]))
    return np.array(sorted(s))


def full_check(cfg, n_sample=None, seed=None, inp=None):
    """Run the GPU layer on seeded inputs and compare it with the oracle.  Returns a report."""
    name = cfg.get("name", "custom")
    say(f"[gpu] {name}: N={cfg['n_tokens']} G={cfg['n_groups']} M={cfg['d_model']} "
        f"H={cfg['d_ff']} E={cfg['n_experts']}+{cfg['n_shared']} k={cfg['top_k']} "
        f"C={cfg['capacity']} dtype={cfg['dtype']} seed={cfg.get('seed', 0) if seed is None else seed}")
    inp = synth.make_inputs(cfg, seed) if inp is None else inp
    dev = to_device(inp, cfg)
    say(f"[gpu] {name}: moe_forward")
    g = run_gpu(cfg, dev)
    say(f"[gpu] {name}: oracle")
    ref_logits = mo.router_logits(inp.x, inp.Wg, inp.bg)
    lerr = rel_err(g["logits"], ref_logits)
    assert lerr <= LOGIT_TOL, f"logits rel err {lerr}"
    ref = mo.route(cfg, g["logits"], inp.u)
    margin = rr_margin(cfg, g["logits"], ref["topk_idx"], inp.u)
    assert margin > 1e-12, f"random-routing decision within {margin} of its threshold"
    check_routing(cfg, g, ref)
    toks = sample_tokens(cfg, ref, n_sample)
    y_ref = mo.layer_outputs(cfg, inp.x, inp.W1, inp.W2, ref, tokens=toks)
    yerr = rel_err(g["y"][toks], y_ref)
    assert yerr <= Y_TOL[cfg["dtype"]], f"y rel err {yerr}"
    dropped = np.nonzero(~(ref["pos"] >= 0).any(axis=1))[0]
    if cfg["residual"] and cfg["n_shared"] == 0 and dropped.size:
        assert (g["y"][dropped] == inp.x[dropped]).all(), "dropped tokens must pass x through"
    rep = dict(name=name, logits_err=lerr, y_err=yerr, aux=g["aux"], aux_ref=ref["aux"],
               z_loss=g["z_loss"], z_loss_ref=ref["z_loss"], dev_loss=g["dev_loss"],
               dev_loss_ref=ref["dev_loss"],
               stats=g["stats"].tolist(), sampled=len(toks), rr_margin=margin)
    say(f"[gpu] {name}: ok {rep}")
    return rep, g, ref, inp, dev
