"""Host-side tests of the C ABI library (no GPU needed, nothing is launched).

The library must load, export every function include/moe.h declares, report its version,
size workspaces, and reject bad arguments on the host with the documented codes before any
HIP call is made.
"""
import ctypes
import os
import re
import subprocess

import pytest

from mixture_experts_layer_group_amd import binding, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from mixture_experts_layer_group_amd import build
        build.build(verbose=False)
    return binding.load_library()


def test_exports_every_declared_symbol(lib):
    declared = binding.header_functions()
    assert {"moe_forward", "moe_route", "moe_workspace_size", "moe_strerror",
            "moe_abi_version", "moe_forward_timed", "moe_backward",
            "moe_backward_workspace_size", "moe_forward_noalloc", "moe_forward_train",
            "moe_backward_saved"} <= set(declared)
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    for name in declared:
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_strerror(lib):
    hdr = open(binding.HEADER).read()
    assert int(re.search(r"#define MOE_ABI_VERSION (\d+)", hdr).group(1)) == binding.moe_abi_version()
    for code in (0, -1, -2, -3, -4, -5, 99):
        assert isinstance(binding.moe_strerror(code), str) and binding.moe_strerror(code)
    assert binding.moe_strerror(-2) != binding.moe_strerror(-1)


def test_workspace_sizes(lib):
    for name, cfg in configs.ALL.items():
        n = binding.moe_workspace_size(cfg)
        assert n > 0
        bigger = dict(cfg, n_tokens=cfg["n_tokens"] * 2)
        assert binding.moe_workspace_size(bigger) >= n
    assert binding.moe_workspace_size(dict(configs.SMALL["small_top2_rr"], n_tokens=0,
                                           n_groups=1)) > 0


BAD = [
    (dict(n_groups=0), binding.MOE_EINVAL),
    (dict(n_tokens=1535), binding.MOE_EINVAL),          # N % G != 0
    (dict(n_tokens=-3, n_groups=1), binding.MOE_EINVAL),
    (dict(top_k=0), binding.MOE_EINVAL),
    (dict(top_k=9, n_experts=16, random_routing=0), binding.MOE_EUNSUPPORTED),
    (dict(top_k=17, n_experts=16, random_routing=0), binding.MOE_EINVAL),
    (dict(n_experts=257, top_k=2), binding.MOE_EUNSUPPORTED),
    (dict(capacity=0), binding.MOE_EINVAL),
    (dict(act=3), binding.MOE_EINVAL),
    (dict(gate_norm=3), binding.MOE_EINVAL),
    (dict(gate_norm=2, norm_p=0.0), binding.MOE_EINVAL),
    (dict(gate_norm=2, norm_p=-1.0), binding.MOE_EINVAL),
    (dict(gate_norm=2, norm_p=float("nan")), binding.MOE_EINVAL),
    (dict(gate_norm=2, norm_p=float("inf")), binding.MOE_EINVAL),
    (dict(expert_groups=0), binding.MOE_EINVAL),
    (dict(expert_groups=3), binding.MOE_EINVAL),                    # E = 8 % 3 != 0
    (dict(expert_groups=4, topk_groups=5), binding.MOE_EINVAL),
    (dict(expert_groups=4, topk_groups=0), binding.MOE_EINVAL),
    (dict(expert_groups=8, topk_groups=1), binding.MOE_EINVAL),     # k = 2 > 1 * 8/8
    (dict(n_experts=128, expert_groups=64, topk_groups=2), binding.MOE_EUNSUPPORTED),
    (dict(random_routing=1, top_k=1), binding.MOE_EINVAL),
    (dict(residual=2), binding.MOE_EINVAL),
    (dict(dtype=5), binding.MOE_EINVAL),
    (dict(d_model=200), binding.MOE_EUNSUPPORTED),       # bf16 needs M % 128 == 0
    (dict(d_ff=320), binding.MOE_EUNSUPPORTED),
    (dict(dtype=0, d_model=96), binding.MOE_EUNSUPPORTED),
    (dict(n_shared=-1), binding.MOE_EINVAL),
    # x of 2 GiB: GEMM 1 gathers rows from all of x through one 32-bit buffer range
    (dict(n_tokens=1 << 22, n_groups=2), binding.MOE_EUNSUPPORTED),
    (dict(n_tokens=1 << 21, n_groups=2, dtype=0), binding.MOE_EUNSUPPORTED),
]


def test_largest_x_under_the_buffer_range_is_accepted(lib):
    # bf16 x of 2^31 - 1024 bytes, one token short of the 32-bit buffer range
    cfg = dict(configs.SMALL["small_top2_rr"], n_tokens=(1 << 22) - 2, n_groups=2)
    assert binding.moe_workspace_size(cfg) > 0


@pytest.mark.parametrize("patch,code", BAD, ids=[str(p) for p, _ in BAD])
def test_bad_cfg_rejected(lib, patch, code):
    cfg = dict(configs.SMALL["small_top2_rr"], **patch)
    with pytest.raises(binding.MoeError) as ei:
        binding.moe_workspace_size(cfg)
    assert ei.value.code == code


class FakeTensor:
    """Stands in for a device tensor: only an address, never dereferenced by these tests."""

    def __init__(self, addr, n=1 << 30):
        self.addr, self.n = addr, n

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n


def _fake_meta(base=0x10000000, bad=None):
    kw = {f: FakeTensor(base + 0x1000 * i) for i, f in enumerate(binding.Meta.FIELDS)}
    if bad:
        kw[bad] = FakeTensor(kw[bad].addr + 4)
    return binding.Meta(**kw)


def _call(cfg, fn="moe_forward", **over):
    wsz = (binding.moe_backward_workspace_size if fn == "moe_forward_train"
           else binding.moe_workspace_size)(cfg)
    a = dict(x=FakeTensor(0x20000000), Wg=FakeTensor(0x21000000), bg=None,
              W1=FakeTensor(0x22000000), W2=FakeTensor(0x23000000), u=FakeTensor(0x24000000),
              y=FakeTensor(0x25000000), aux=FakeTensor(0x26000000), meta=_fake_meta(),
              ws=FakeTensor(0x27000000, wsz))
    a.update(over)
    getattr(binding, fn)(cfg, a["x"], a["Wg"], a["bg"], a["W1"], a["W2"], a["u"], a["y"],
                         a["aux"], a["meta"], a["ws"], stream=_NoStream())


class _NoStream:
    cuda_stream = 0


INVALID_CALLS = [
    ("null x", dict(x=FakeTensor(0)), binding.MOE_EINVAL),
    ("misaligned W1", dict(W1=FakeTensor(0x22000008)), binding.MOE_EINVAL),
    ("null y", dict(y=FakeTensor(0)), binding.MOE_EINVAL),
    ("misaligned aux", dict(aux=FakeTensor(0x26000004)), binding.MOE_EINVAL),
    ("null u with random routing", dict(u=None), binding.MOE_EINVAL),
    ("misaligned bg", dict(bg=FakeTensor(0x28000002)), binding.MOE_EINVAL),
    ("misaligned meta.row", dict(meta=_fake_meta(bad="row")), binding.MOE_EINVAL),
    ("misaligned meta.z_loss", dict(meta=_fake_meta(bad="z_loss")), binding.MOE_EINVAL),
    ("misaligned meta.dev_loss", dict(meta=_fake_meta(bad="dev_loss")), binding.MOE_EINVAL),
    ("null meta.logits", dict(meta=binding.Meta(**{f: FakeTensor(0x10000000 + 0x1000 * i)
                                                   for i, f in enumerate(binding.Meta.FIELDS)
                                                   if f != "logits"})), binding.MOE_EINVAL),
    ("small workspace", dict(ws=FakeTensor(0x27000000, 1024)), binding.MOE_EWORKSPACE),
    ("null workspace", dict(ws=FakeTensor(0, 1 << 30)), binding.MOE_EINVAL),
]


@pytest.mark.parametrize("fn", ["moe_forward", "moe_forward_train"])
@pytest.mark.parametrize("what,over,code", INVALID_CALLS, ids=[w for w, _, _ in INVALID_CALLS])
def test_invalid_forward_rejected_on_host(lib, what, over, code, fn):
    """Each call fails its host checks, so nothing is enqueued (no GPU is touched)."""
    cfg = configs.SMALL["small_top2_rr"]
    with pytest.raises(binding.MoeError) as ei:
        _call(cfg, fn, **over)
    assert ei.value.code == code, what


def test_train_forward_needs_the_backward_workspace(lib):
    """moe_forward_train keeps activations in the backward's workspace: a forward-sized one
    is refused, for every workload (the backward workspace is strictly larger)."""
    for cfg in list(configs.SMALL.values()) + list(configs.WORKLOADS.values()):
        ws = FakeTensor(0x27000000, binding.moe_workspace_size(cfg))
        with pytest.raises(binding.MoeError) as ei:
            _call(cfg, "moe_forward_train", ws=ws)
        assert ei.value.code == binding.MOE_EWORKSPACE, cfg["name"]


def test_invalid_route_rejected_on_host(lib):
    cfg = configs.SMALL["small_top2_rr"]
    ws = FakeTensor(0x27000000, binding.moe_workspace_size(cfg))
    for over, code in ((dict(logits=FakeTensor(0)), binding.MOE_EINVAL),
                       (dict(u=None), binding.MOE_EINVAL),
                       (dict(ws=FakeTensor(0x27000000, 16)), binding.MOE_EWORKSPACE)):
        a = dict(logits=FakeTensor(0x30000000), u=FakeTensor(0x24000000), ws=ws)
        a.update(over)
        with pytest.raises(binding.MoeError) as ei:
            binding.moe_route(cfg, a["logits"], a["u"], _fake_meta(), FakeTensor(0x26000000),
                              a["ws"], stream=_NoStream())
        assert ei.value.code == code


def test_null_cfg_rejected(lib):
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_size(None, ctypes.byref(n)) == binding.MOE_EINVAL
    assert lib.moe_forward(None, *([None] * 9), None, 0, None) == binding.MOE_EINVAL


def _bwd_call(cfg, fn="moe_backward", **over):
    a = dict(x=FakeTensor(0x20000000), Wg=FakeTensor(0x21000000), bg=None,
             W1=FakeTensor(0x22000000), W2=FakeTensor(0x23000000), u=FakeTensor(0x24000000),
             dy=FakeTensor(0x25000000), coefs=(0.1, 0.01, 0.0), dx=FakeTensor(0x29000000),
             dWg=FakeTensor(0x2a000000), dbg=None, dW1=FakeTensor(0x2b000000),
             dW2=FakeTensor(0x2c000000), meta=_fake_meta(),
             ws=FakeTensor(0x27000000, binding.moe_backward_workspace_size(cfg)))
    a.update(over)
    getattr(binding, fn)(cfg, a["x"], a["Wg"], a["bg"], a["W1"], a["W2"], a["u"], a["dy"],
                         *a["coefs"], a["dx"], a["dWg"], a["dbg"], a["dW1"], a["dW2"], a["meta"],
                         a["ws"], stream=_NoStream())


INVALID_BWD = [
    ("null dy", dict(dy=FakeTensor(0)), binding.MOE_EINVAL),
    ("null dx", dict(dx=FakeTensor(0)), binding.MOE_EINVAL),
    ("misaligned dW1", dict(dW1=FakeTensor(0x2b000004)), binding.MOE_EINVAL),
    ("null dWg", dict(dWg=FakeTensor(0)), binding.MOE_EINVAL),
    ("misaligned dbg", dict(dbg=FakeTensor(0x2d000008)), binding.MOE_EINVAL),
    ("nan coefficient", dict(coefs=(float("nan"), 0.0, 0.0)), binding.MOE_EINVAL),
    ("inf coefficient", dict(coefs=(0.0, float("inf"), 0.0)), binding.MOE_EINVAL),
    ("forward-sized workspace", dict(ws=FakeTensor(0x27000000, 4096)), binding.MOE_EWORKSPACE),
    ("null u with random routing", dict(u=None), binding.MOE_EINVAL),
    ("misaligned meta.pos", dict(meta=_fake_meta(bad="pos")), binding.MOE_EINVAL),
]


@pytest.mark.parametrize("fn", ["moe_backward", "moe_backward_saved"])
@pytest.mark.parametrize("what,over,code", INVALID_BWD, ids=[w for w, _, _ in INVALID_BWD])
def test_invalid_backward_rejected_on_host(lib, what, over, code, fn):
    cfg = configs.SMALL["small_top2_rr"]
    with pytest.raises(binding.MoeError) as ei:
        _bwd_call(cfg, fn, **over)
    assert ei.value.code == code, what


def test_backward_workspace_covers_forward(lib):
    for cfg in list(configs.SMALL.values()) + list(configs.WORKLOADS.values()):
        assert binding.moe_backward_workspace_size(cfg) > binding.moe_workspace_size(cfg)


def test_backward_workspace_sizes_small_batches(lib):
    # the token-range split of the router weight gradient must handle every batch size,
    # the empty batch included (no token range at all)
    base = configs.SMALL["small_top2_rr"]
    for n in (0, 1, 127, 128, 129, 4096):
        cfg = configs.with_overrides(base, n_tokens=n, n_groups=1)
        assert binding.moe_backward_workspace_size(cfg) > 0, n


# ---- moe_forward_noalloc: host-side checks (the scratch array is never touched here)

def test_noalloc_scratch_size_matches_header(lib):
    hdr = open(binding.HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.MOE_NOALLOC_SCRATCH_BYTES


def _noalloc_call(cfg, **over):
    a = dict(x=FakeTensor(0x20000000), Wg=FakeTensor(0x21000000), bg=None,
             W1=FakeTensor(0x22000000), W2=FakeTensor(0x23000000), u=FakeTensor(0x24000000),
             y=FakeTensor(0x25000000), aux=FakeTensor(0x26000000), meta=_fake_meta())
    a.update(over)
    binding.moe_forward_noalloc(cfg, a["x"], a["Wg"], a["bg"], a["W1"], a["W2"], a["u"],
                                a["y"], a["aux"], a["meta"], stream=_NoStream())


NOALLOC_BAD = [
    ("bad cfg", dict(n_groups=0), {}, binding.MOE_EINVAL),
    ("unsupported cfg", dict(d_model=200), {}, binding.MOE_EUNSUPPORTED),
    # the GShard-style layer needs 0.3 GB of workspace
    ("larger than the scratch", dict(configs.WORKLOADS["gshard_bf16"]), {}, binding.MOE_ESCRATCH),
    ("null x", {}, dict(x=FakeTensor(0)), binding.MOE_EINVAL),
    ("misaligned aux", {}, dict(aux=FakeTensor(0x26000004)), binding.MOE_EINVAL),
    ("null u with random routing", {}, dict(u=None), binding.MOE_EINVAL),
    ("misaligned meta.pos", {}, dict(meta=_fake_meta(bad="pos")), binding.MOE_EINVAL),
]


@pytest.mark.parametrize("what,patch,over,code", NOALLOC_BAD, ids=[w for w, _, _, _ in NOALLOC_BAD])
def test_noalloc_rejected_on_host(lib, what, patch, code, over):
    cfg = dict(configs.SMALL["small_top2_rr"], **patch)
    with pytest.raises(binding.MoeError) as ei:
        _noalloc_call(cfg, **over)
    assert ei.value.code == code, what


def test_noalloc_limit_is_the_forward_workspace(lib):
    """A layer is accepted by moe_forward_noalloc iff its forward workspace fits the scratch."""
    base = configs.SMALL["small_top2_rr"]
    for n in (1536, 3 * 4096, 3 * 16384, 3 * 65536):
        cfg = configs.with_overrides(base, n_tokens=n, capacity=n // 24)
        fits = binding.moe_workspace_size(cfg) <= binding.MOE_NOALLOC_SCRATCH_BYTES
        if not fits:
            with pytest.raises(binding.MoeError) as ei:
                _noalloc_call(cfg)
            assert ei.value.code == binding.MOE_ESCRATCH
