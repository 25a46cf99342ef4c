"""moe_forward_noalloc (the forward on the library's static per-GPU scratch) against
moe_forward with a caller-allocated workspace, through the C ABI.

Both run the same kernels on the same inputs, so every output must match bit for bit: y, the
logits, routing, positions, rows, counts, offsets, stats, aux, z-loss and device loss.  Two
calls in a row, the second with a smaller layer (the scratch then holds the first call's
contents), and the first layer once more after it.
"""
import numpy as np
import pytest

from mixture_experts_layer_group_amd import binding, configs, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# A GShard-style layer near the scratch size (about 45 MB of forward workspace: 4096 kept rows
# of M = 1024 and H = 4096), then a small layer with shared SwiGLU experts.
LARGE = configs.with_overrides(configs.WORKLOADS["gshard_bf16"], name="noalloc_large",
                               n_tokens=2048, n_groups=1, capacity=64)
SMALL = configs.SMALL["small_swiglu_shared"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _inputs(cfg):
    import gpu_harness
    return gpu_harness.to_device(synth.make_inputs(cfg), cfg)


def _run(cfg, dev, noalloc):
    meta = binding.alloc_meta(cfg)
    for t in (meta.logits, meta.topk_w, meta.z_loss, meta.dev_loss):
        t.fill_(float("nan"))
    for t in (meta.topk_idx, meta.pos, meta.row, meta.count, meta.offset, meta.stats):
        t.fill_(-7)
    y = torch.full_like(dev["x"], float("nan"))
    aux = torch.full((4,), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        binding.moe_forward_noalloc(cfg, dev["x"], dev["Wg"], dev["bg"], dev["W1"], dev["W2"],
                                    dev["u"], y, aux, meta)
    else:
        ws = binding.alloc_workspace(cfg)
        binding.moe_forward(cfg, dev["x"], dev["Wg"], dev["bg"], dev["W1"], dev["W2"],
                            dev["u"], y, aux, meta, ws)
    torch.cuda.synchronize()
    out = meta.to_numpy()
    out["y"] = y.view(torch.int16).cpu().numpy() if y.dtype == torch.bfloat16 else \
        y.view(torch.int32).cpu().numpy()
    out["aux"] = aux[:1].cpu().numpy()
    return out


def _same(a, b, what):
    for f, v in a.items():
        assert np.array_equal(v.view(np.uint8), b[f].view(np.uint8)), f"{what}: {f} differs"


def test_noalloc_matches_forward_twice_in_a_row():
    assert binding.moe_workspace_size(LARGE) <= binding.MOE_NOALLOC_SCRATCH_BYTES
    assert binding.moe_workspace_size(LARGE) > 0.5 * binding.MOE_NOALLOC_SCRATCH_BYTES
    assert binding.moe_workspace_size(SMALL) < binding.moe_workspace_size(LARGE)
    dl, ds = _inputs(LARGE), _inputs(SMALL)
    ref_l = _run(LARGE, dl, noalloc=False)
    ref_s = _run(SMALL, ds, noalloc=False)
    assert ref_l["stats"][0] > 0 and ref_s["stats"][0] > 0
    _same(_run(LARGE, dl, noalloc=True), ref_l, "first call (large layer)")
    _same(_run(SMALL, ds, noalloc=True), ref_s, "second call (smaller layer)")
    _same(_run(LARGE, dl, noalloc=True), ref_l, "third call (large layer again)")


def test_noalloc_rejects_a_layer_beyond_the_scratch():
    cfg = configs.WORKLOADS["gshard_bf16"]
    dev = _inputs(configs.with_overrides(cfg, n_tokens=8, n_groups=1))   # pointers only
    meta = binding.alloc_meta(configs.with_overrides(cfg, n_tokens=8, n_groups=1))
    aux = torch.empty(4, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.MoeError) as ei:
        binding.moe_forward_noalloc(cfg, dev["x"], dev["Wg"], dev["bg"], dev["W1"], dev["W2"],
                                    dev["u"], dev["x"], aux, meta)
    assert ei.value.code == binding.MOE_ESCRATCH
