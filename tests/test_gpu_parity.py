"""GPU parity of the HIP MoE layer against the CPU oracle, through the C ABI.

Small layers (several GEMM tiles, ragged expert tails, ragged router blocks, several groups,
every gating flag) and the reference workloads at their full sizes are all compared in full:
routing, positions, rows and aux on every token (bit-exact / 1e-5) and the output y on every
token (1e-4 fp32, 2e-2 bf16).
"""
import numpy as np
import pytest

from mixture_experts_layer_group_amd import binding, configs, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def harness():
    import gpu_harness
    return gpu_harness


@pytest.mark.parametrize("name", sorted(configs.SMALL))
def test_small_layer_parity(name):
    harness().full_check(configs.SMALL[name])


# Every workload's output y is compared on every token against the fp64 oracle (it evaluates
# one expert at a time, so host memory stays bounded; about a minute of host work for all
# seven layers).
@pytest.mark.parametrize("name", list(configs.WORKLOADS))
def test_workload_parity(name):
    rep = harness().full_check(configs.WORKLOADS[name], n_sample=None)[0]
    assert rep["sampled"] == configs.WORKLOADS[name]["n_tokens"]
    if name == "large_expert_bf16":
        assert rep["stats"][1] == 0 and rep["stats"][2] == 0   # dropless


def test_route_from_oracle_logits():
    """Reverse direction: moe_route fed the oracle's own logits (rounded to fp32)."""
    h = harness()
    from oracle import moe_oracle as mo
    for name in ("small_top2_rr", "small_shared_top3", "small_pnorm_top4", "small_grouped_top4",
                 "gshard_bf16"):
        cfg = configs.ALL[name]
        h.say(f"[gpu] moe_route {name}")
        inp = synth.make_inputs(cfg)
        l32 = mo.router_logits(inp.x, inp.Wg, inp.bg).astype(np.float32)
        ref = mo.route(cfg, l32, inp.u)
        meta = binding.alloc_meta(cfg)
        ws = binding.alloc_workspace(cfg)
        aux = torch.empty(4, dtype=torch.float32, device="cuda")
        u = torch.from_numpy(inp.u).cuda() if inp.u is not None else None
        binding.moe_route(cfg, torch.from_numpy(l32).cuda(), u, meta, aux, ws)
        torch.cuda.synchronize()
        g = meta.to_numpy()
        g["aux"] = float(aux[0].cpu())
        g["z_loss"] = float(g["z_loss"][0])
        g["dev_loss"] = float(g["dev_loss"][0])
        h.check_routing(cfg, g, ref)


def test_deterministic_and_padding_never_read():
    """Three runs are bitwise identical, also when the workspace starts as all-NaN bytes
    (unfilled capacity rows and tile padding are never read into y)."""
    h = harness()
    cfg = configs.SMALL["small_shared_top3"]
    inp = synth.make_inputs(cfg)
    dev = h.to_device(inp, cfg)
    ws = binding.alloc_workspace(cfg)
    outs = []
    for fill in (0, 0xFF, 0x7F):
        ws.fill_(fill)
        outs.append(h.run_gpu(cfg, dev, workspace=ws))
    for o in outs[1:]:
        for f in ("y", "logits", "topk_idx", "topk_w", "pos", "row", "count", "offset", "stats"):
            assert np.array_equal(o[f], outs[0][f], equal_nan=False), f
        for f in ("aux", "z_loss", "dev_loss"):
            assert o[f] == outs[0][f], f
    assert np.isfinite(outs[0]["y"]).all()


def _cfg(**kw):
    base = dict(name="edge", n_tokens=256, n_groups=1, d_model=128, d_ff=128, n_experts=4,
                n_shared=0, top_k=2, capacity=128, act=0, gate_norm=1, random_routing=0,
                residual=1, dtype=1, zipf_s=0.0, seed=21)
    base.update(kw)
    return base


EDGE = {
    "capacity_one": _cfg(capacity=1, n_groups=4),
    "k_equals_E": _cfg(n_experts=4, top_k=4, capacity=256),
    "one_token_groups": _cfg(n_tokens=96, n_groups=96, capacity=1, n_experts=6),
    "max_experts_topk8": _cfg(n_tokens=640, n_experts=256, top_k=8, capacity=24, d_model=256,
                              d_ff=256, act=1),
    "single_expert_k1": _cfg(n_experts=1, top_k=1, capacity=256, gate_norm=0),
    "fp32_ragged": _cfg(dtype=0, n_tokens=333, n_experts=7, top_k=3, capacity=50, d_model=64,
                        d_ff=192, act=1),
    "bare_layer_drops": _cfg(residual=0, capacity=20, n_experts=8, zipf_s=1.5),
    "one_token": _cfg(n_tokens=1, capacity=1),
    "pnorm_p8_top8": _cfg(n_experts=32, top_k=8, capacity=64, gate_norm=2, norm_p=8.0,
                          n_groups=2),
    "grouped_fp32": _cfg(dtype=0, n_tokens=330, n_experts=12, top_k=3, capacity=60,
                         d_model=64, d_ff=128, expert_groups=4, topk_groups=2, n_groups=3),
    "grouped_32_groups_top8": _cfg(n_tokens=640, n_experts=256, top_k=8, capacity=24,
                                   d_model=256, d_ff=256, expert_groups=32, topk_groups=4,
                                   zipf_s=0.5),
    "grouped_one_group": _cfg(n_experts=16, top_k=4, capacity=100, expert_groups=4,
                              topk_groups=1, act=2),
    # rows of more than 1024 16-byte chunks: one token per combine block and several load
    # rounds per lane; GEMM 1 over K = 9216 with a half-filled n-tile (d_ff = 128)
    "wide_rows_bf16": _cfg(n_tokens=300, d_model=9216, d_ff=128, n_experts=4, capacity=60,
                           act=1, n_groups=2),
    "wide_rows_fp32": _cfg(dtype=0, n_tokens=200, d_model=4160, d_ff=64, n_experts=3,
                           top_k=2, capacity=90, act=1),
    # more 64-token router blocks than the chip has CUs: the router's two-blocks-per-CU form
    # (8 lanes per token), with 32 expert groups (four per lane) and with random routing
    "pair_router_grouped": _cfg(n_tokens=16640, n_experts=128, top_k=4, capacity=700,
                                expert_groups=32, topk_groups=4, act=2, zipf_s=0.7),
    "pair_router_random": _cfg(n_tokens=16448, n_groups=4, n_experts=64, top_k=2,
                               capacity=150, random_routing=1, act=1),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_case_parity(name):
    harness().full_check(dict(EDGE[name], name=name))


def test_all_tokens_same_preference():
    """Every token ranks experts 0 > 1 > 2 > 3 (router offsets dominate): count = [C, C, 0, 0]
    and tokens C..S-1 are fully dropped, passing x through bit-exactly."""
    h = harness()
    cfg = _cfg(name="same_pref")
    inp = synth.make_inputs(cfg)
    inp.bg = np.array([300.0, 200.0, 100.0, 0.0], np.float32)
    rep, g, ref, inp, dev = h.full_check(cfg, inp=inp)
    assert g["count"].tolist() == [[128, 128, 0, 0]]
    assert g["stats"].tolist() == [256, 256, 128, 0]
    assert (g["y"][128:] == inp.x[128:]).all()


def test_empty_batch():
    cfg = _cfg(n_tokens=0)
    meta = binding.alloc_meta(cfg)
    meta.count.fill_(7)
    meta.offset.fill_(7)
    meta.stats.fill_(7)
    meta.z_loss.fill_(7)
    meta.dev_loss.fill_(7)
    ws = binding.alloc_workspace(cfg)
    aux = torch.full((4,), 5.0, device="cuda")
    empty = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    binding.moe_forward(cfg, empty, None, None, None, None, None, empty, aux, meta, ws)
    torch.cuda.synchronize()
    assert int(meta.count.abs().sum()) == 0 and int(meta.offset.abs().sum()) == 0
    assert int(meta.stats.abs().sum()) == 0 and float(aux[0]) == 0.0
    assert float(meta.z_loss[0]) == 0.0 and float(meta.dev_loss[0]) == 0.0


# (act, n_tokens, d_model, d_ff).  The larger shapes give each GEMM more 256 x 256 tiles than
# the chip has compute units, so blocks of the persistent bf16 kernel run several tiles, with
# a ragged last m-tile and a partial last n-tile; d_model = 256 makes GEMM 1's K loop (4
# chunks) shorter than the deferred stores of the previous tile.
DENSE = {"gelu_small": (1, 700, 256, 384), "swiglu_small": (2, 700, 256, 384),
         "relu_multi_tile": (0, 16461, 1152, 1152), "gelu_short_k": (1, 16461, 256, 1152),
         "swiglu_multi_tile": (2, 16461, 1152, 1152), "swiglu_short_k": (2, 16461, 256, 1408)}


@pytest.mark.parametrize("case", list(DENSE))
def test_single_expert_is_a_dense_ffn(case):
    """E=1, k=1, C=N, norm=none: y = x + act(x W1^T) W2^T (gated: (silu(x G^T) * x U^T)
    W2^T), checked against torch.matmul and torch's relu / gelu / silu in fp32 on the GPU
    (library routines) rather than against the oracle."""
    act, n, dm, dff = DENSE[case]
    cfg = _cfg(n_tokens=n, n_experts=1, top_k=1, capacity=n, gate_norm=0, act=act,
               d_model=dm, d_ff=dff)
    inp = synth.make_inputs(cfg)
    h = harness()
    dev = h.to_device(inp, cfg)
    g = h.run_gpu(cfg, dev)
    x = dev["x"].float()
    w1 = dev["W1"][0].float().contiguous()
    w2 = dev["W2"][0].float().contiguous()
    pre = torch.matmul(x, w1.t().contiguous())
    if act == 0:
        hid = torch.relu(pre)
    elif act == 1:
        hid = torch.nn.functional.gelu(pre)
    else:
        H = cfg["d_ff"]
        hid = torch.nn.functional.silu(pre[:, :H]) * pre[:, H:]
    ref = (x + torch.matmul(hid, w2.t().contiguous())).cpu().numpy()
    assert h.rel_err(g["y"], ref) <= 2e-2
