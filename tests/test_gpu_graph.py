"""moe_forward and moe_backward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing, issues no memset and never synchronises, so one call can be
recorded into a graph.  Each replay is compared bit for bit with the eager result (the layer
is deterministic), with the outputs poisoned before every replay (and the forward's workspace
refilled with the byte patterns its determinism test uses) and other eager calls of the
library in between.
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


META = ("logits", "topk_idx", "topk_w", "pos", "row", "count", "offset", "stats", "z_loss")


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _poison(tensors):
    for t in tensors:
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


@pytest.mark.parametrize("name", ["small_top2_rr", "small_swiglu_shared", "small_grouped_top4"])
def test_forward_graph_replays_match_eager(name):
    cfg = configs.SMALL[name]
    h = harness()
    h.say(f"[gpu] graph forward {name}")
    dev = h.to_device(synth.make_inputs(cfg), cfg)
    args = (dev["x"], dev["Wg"], dev["W1"], dev["W2"])
    y_ref, aux_ref, meta_ref = binding.forward(cfg, *args, bg=dev["bg"], u=dev["u"])
    torch.cuda.synchronize()
    ref = {"y": y_ref.clone(), "aux": aux_ref.clone()}
    ref.update({k: getattr(meta_ref, k).clone() for k in META})

    meta = binding.alloc_meta(cfg)
    y = torch.empty_like(dev["x"])
    aux = torch.empty((4,), dtype=torch.float32, device="cuda")
    ws = binding.alloc_workspace(cfg)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # one call on the capture's stream type before capture
        binding.moe_forward(cfg, *args[:2], dev["bg"], *args[2:], dev["u"], y, aux, meta, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.moe_forward(cfg, *args[:2], dev["bg"], *args[2:], dev["u"], y, aux, meta, ws)
    torch.cuda.synchronize()
    outs = [y, aux] + [getattr(meta, k) for k in META]
    for r in range(4):
        _poison(outs)
        ws.fill_(0xFF if r % 2 else 0x7F)   # the workspace's earlier contents are never read
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {"y": y, "aux": aux[:1]}
        got.update({k: getattr(meta, k) for k in META})
        for k, v in ref.items():
            a, b = (got[k][:1], v[:1]) if k == "z_loss" else (got[k], v)
            assert np.array_equal(_bytes(a), _bytes(b)), f"replay {r}: {k} differs"
        # eager use of the library between replays, on other buffers
        binding.forward(cfg, *args, bg=dev["bg"], u=dev["u"])
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["small_top2_rr", "small_swiglu_shared"])
def test_backward_graph_replays_match_eager(name):
    cfg = configs.SMALL[name]
    h = harness()
    h.say(f"[gpu] graph backward {name}")
    dev = h.to_device(synth.make_inputs(cfg), cfg)
    gen = torch.Generator(device="cpu").manual_seed(5)
    dy = torch.randn(tuple(dev["x"].shape), generator=gen).to(dev["x"].dtype).cuda()
    args = (dev["x"], dev["Wg"], dev["W1"], dev["W2"], dy)
    coefs = dict(coef_aux=0.5, coef_z=0.25, coef_dev=0.0)
    ref, _ = binding.backward(cfg, *args, bg=dev["bg"], u=dev["u"], **coefs)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items()}

    f32 = dict(dtype=torch.float32, device="cuda")
    out = dict(dx=torch.empty_like(dev["x"]), dWg=torch.empty(tuple(dev["Wg"].shape), **f32),
               dbg=torch.empty((cfg["n_experts"],), **f32),
               dW1=torch.empty(tuple(dev["W1"].shape), **f32),
               dW2=torch.empty(tuple(dev["W2"].shape), **f32))
    meta = binding.alloc_meta(cfg)
    ws = torch.empty(max(1, binding.moe_backward_workspace_size(cfg)), dtype=torch.uint8,
                     device="cuda")

    def call():
        binding.moe_backward(cfg, dev["x"], dev["Wg"], dev["bg"], dev["W1"], dev["W2"],
                             dev["u"], dy, coefs["coef_aux"], coefs["coef_z"],
                             coefs["coef_dev"], out["dx"], out["dWg"], out["dbg"],
                             out["dW1"], out["dW2"], meta, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        _poison(list(out.values()))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert np.array_equal(_bytes(out[k]), _bytes(v)), f"replay {r}: {k} differs"
        binding.backward(cfg, *args, bg=dev["bg"], u=dev["u"], **coefs)
        torch.cuda.synchronize()
