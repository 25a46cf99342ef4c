"""ctypes binding of libmoe.so (include/moe.h).  Argument marshalling only.

Every step of the layer runs in the HIP library; this module turns torch tensors into
device pointers, allocates outputs and workspace with ``torch.empty`` and passes torch's
current HIP stream.  If libmoe.so is missing it raises: there is no fallback path.
"""
import ctypes
import os
import re

from .configs import CFG_FIELDS

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_EWORKSPACE, MOE_EUNSUPPORTED, MOE_EHIP, MOE_ESCRATCH = 0, -1, -2, -3, -4, -5
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_N_EVENTS = 7
STAGES = ("router", "gate", "permute", "ffn1", "ffn2", "combine")


_FLOAT_FIELDS = ("norm_p",)


class MoeCfg(ctypes.Structure):
    _fields_ = [(f, ctypes.c_float if f in _FLOAT_FIELDS else ctypes.c_int32)
                for f in CFG_FIELDS]


META_FIELDS = ("logits", "topk_idx", "topk_w", "pos", "row", "count", "offset", "stats",
               "z_loss", "dev_loss")
# moe_cfg fields a workload dict may leave out, and the values that turn them off
CFG_DEFAULTS = {"norm_p": 1.0, "expert_groups": 1, "topk_groups": 1}


class MoeMetaC(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in META_FIELDS]


class MoeError(RuntimeError):
    def __init__(self, code, where):
        super().__init__(f"{where}: {moe_strerror(code)} ({code})")
        self.code = code


_lib = None


def load_library(path=LIB_PATH):
    """Load libmoe.so (cached).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m mixture_experts_layer_group_amd.build`")
    # torch ships its own HIP runtime under the same soname as ROCm's: load it first, so that
    # libmoe.so binds to the runtime that owns torch's streams, events and allocations (loaded
    # the other way round, the process ends up mixing two runtimes and launches fail)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    cfgp, metap = ctypes.POINTER(MoeCfg), ctypes.POINTER(MoeMetaC)
    lib.moe_abi_version.restype = i32
    lib.moe_abi_version.argtypes = []
    lib.moe_strerror.restype = ctypes.c_char_p
    lib.moe_strerror.argtypes = [i32]
    lib.moe_workspace_size.restype = i32
    lib.moe_workspace_size.argtypes = [cfgp, ctypes.POINTER(sz)]
    fwd = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, metap, vp, sz, vp]
    lib.moe_forward.restype = i32
    lib.moe_forward.argtypes = fwd
    lib.moe_forward_timed.restype = i32
    lib.moe_forward_timed.argtypes = fwd + [ctypes.POINTER(vp)]
    lib.moe_forward_noalloc.restype = i32
    lib.moe_forward_noalloc.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, metap, vp]
    lib.moe_backward_workspace_size.restype = i32
    lib.moe_backward_workspace_size.argtypes = [cfgp, ctypes.POINTER(sz)]
    f32 = ctypes.c_float
    bwd = [cfgp, vp, vp, vp, vp, vp, vp, vp, f32, f32, f32, vp, vp, vp, vp, vp, metap, vp, sz, vp]
    lib.moe_backward.restype = i32
    lib.moe_backward.argtypes = bwd
    lib.moe_forward_train.restype = i32
    lib.moe_forward_train.argtypes = fwd
    lib.moe_backward_saved.restype = i32
    lib.moe_backward_saved.argtypes = bwd
    lib.moe_route.restype = i32
    lib.moe_route.argtypes = [cfgp, vp, vp, metap, vp, vp, sz, vp]
    _lib = lib
    return lib


def header_functions(path=HEADER):
    """Names of the functions include/moe.h declares."""
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, re.M)))


def moe_abi_version():
    return load_library().moe_abi_version()


def moe_strerror(code):
    return load_library().moe_strerror(int(code)).decode()


def make_cfg(cfg):
    """dict (configs.py style) or MoeCfg -> MoeCfg."""
    if isinstance(cfg, MoeCfg):
        return cfg
    def val(f):
        v = cfg[f] if f in cfg else CFG_DEFAULTS[f]
        return float(v) if f in _FLOAT_FIELDS else int(v)
    return MoeCfg(**{f: val(f) for f in CFG_FIELDS})


def moe_workspace_size(cfg):
    n = ctypes.c_size_t(0)
    rc = load_library().moe_workspace_size(ctypes.byref(make_cfg(cfg)), ctypes.byref(n))
    if rc:
        raise MoeError(rc, "moe_workspace_size")
    return n.value


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


class Meta:
    """Device tensors of the dispatch metadata (moe_meta)."""

    FIELDS = META_FIELDS

    def __init__(self, **tensors):
        for f in self.FIELDS:
            setattr(self, f, tensors.get(f))

    def as_struct(self):
        return MoeMetaC(**{f: _ptr(getattr(self, f)) for f in self.FIELDS})

    def to_numpy(self):
        return {f: getattr(self, f).cpu().numpy() for f in self.FIELDS
                if getattr(self, f) is not None}


def alloc_meta(cfg, device="cuda"):
    import torch
    N, E, k, G = cfg["n_tokens"], cfg["n_experts"], cfg["top_k"], cfg["n_groups"]
    i32 = dict(dtype=torch.int32, device=device)
    return Meta(logits=torch.empty((N, E), dtype=torch.float32, device=device),
                topk_idx=torch.empty((N, k), **i32),
                topk_w=torch.empty((N, k), dtype=torch.float32, device=device),
                pos=torch.empty((N, k), **i32), row=torch.empty((N, k), **i32),
                count=torch.empty((G, E), **i32), offset=torch.empty((E + 1,), **i32),
                stats=torch.empty((4,), **i32),
                z_loss=torch.empty((4,), dtype=torch.float32, device=device),
                dev_loss=torch.empty((4,), dtype=torch.float32, device=device))


def moe_backward_workspace_size(cfg):
    n = ctypes.c_size_t(0)
    rc = load_library().moe_backward_workspace_size(ctypes.byref(make_cfg(cfg)), ctypes.byref(n))
    if rc:
        raise MoeError(rc, "moe_backward_workspace_size")
    return n.value


def _backward_call(fn, cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z, coef_dev, dx, dWg,
                   dbg, dW1, dW2, meta, workspace, stream):
    c = make_cfg(cfg)
    m = meta.as_struct()
    rc = getattr(load_library(), fn)(
        ctypes.byref(c), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(W2), _ptr(u), _ptr(dy),
        float(coef_aux), float(coef_z), float(coef_dev), _ptr(dx), _ptr(dWg), _ptr(dbg),
        _ptr(dW1), _ptr(dW2), ctypes.byref(m), _ptr(workspace), workspace.numel(),
        _stream(stream))
    if rc:
        raise MoeError(rc, fn)


def moe_backward(cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z, coef_dev, dx, dWg, dbg, dW1,
                 dW2, meta, workspace, stream=None):
    """C ABI moe_backward on torch tensors (see include/moe.h)."""
    _backward_call("moe_backward", cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z, coef_dev,
                   dx, dWg, dbg, dW1, dW2, meta, workspace, stream)


def moe_backward_saved(cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z, coef_dev, dx, dWg, dbg,
                       dW1, dW2, meta, workspace, stream=None):
    """C ABI moe_backward_saved: the backward on the activations moe_forward_train kept in
    workspace."""
    _backward_call("moe_backward_saved", cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z,
                   coef_dev, dx, dWg, dbg, dW1, dW2, meta, workspace, stream)


def alloc_grads(cfg, x, Wg, W1, W2):
    """Gradient buffers (torch.empty) of moe_backward: dict(dx, dWg, dbg, dW1, dW2)."""
    import torch
    f32 = dict(dtype=torch.float32, device=x.device)
    return dict(dx=torch.empty_like(x), dWg=torch.empty(tuple(Wg.shape), **f32),
                dbg=torch.empty((cfg["n_experts"],), **f32),
                dW1=torch.empty(tuple(W1.shape), **f32), dW2=torch.empty(tuple(W2.shape), **f32))


def alloc_backward_workspace(cfg, device="cuda"):
    import torch
    return torch.empty(max(1, moe_backward_workspace_size(cfg)), dtype=torch.uint8,
                       device=device)


def backward(cfg, x, Wg, W1, W2, dy, bg=None, u=None, coef_aux=0.0, coef_z=0.0, coef_dev=0.0,
             workspace=None, meta=None, stream=None):
    """Allocate the gradients (torch.empty) and run moe_backward.
    Returns dict(dx, dWg, dbg, dW1, dW2) and the meta."""
    meta = alloc_meta(cfg, x.device) if meta is None else meta
    out = alloc_grads(cfg, x, Wg, W1, W2)
    if workspace is None:
        workspace = alloc_backward_workspace(cfg, x.device)
    moe_backward(cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z, coef_dev, out["dx"],
                 out["dWg"], out["dbg"], out["dW1"], out["dW2"], meta, workspace, stream)
    return out, meta


def moe_forward_train(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta, workspace, stream=None):
    """C ABI moe_forward_train: moe_forward into a moe_backward workspace that keeps the
    expert activations for moe_backward_saved."""
    c = make_cfg(cfg)
    m = meta.as_struct()
    rc = load_library().moe_forward_train(
        ctypes.byref(c), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(W2), _ptr(u), _ptr(y),
        _ptr(aux_loss), ctypes.byref(m), _ptr(workspace), workspace.numel(), _stream(stream))
    if rc:
        raise MoeError(rc, "moe_forward_train")


def forward_train(cfg, x, Wg, W1, W2, bg=None, u=None, workspace=None, meta=None, y=None,
                  stream=None):
    """Allocate outputs and a backward workspace, run moe_forward_train.
    Returns (y, aux_loss, meta, workspace); pass meta and workspace to backward_saved."""
    import torch
    dev = x.device
    meta = alloc_meta(cfg, dev) if meta is None else meta
    y = torch.empty_like(x) if y is None else y
    aux = torch.empty((4,), dtype=torch.float32, device=dev)
    workspace = alloc_backward_workspace(cfg, dev) if workspace is None else workspace
    moe_forward_train(cfg, x, Wg, bg, W1, W2, u, y, aux, meta, workspace, stream)
    return y, aux[:1], meta, workspace


def backward_saved(cfg, x, Wg, W1, W2, dy, workspace, meta, bg=None, u=None, coef_aux=0.0,
                   coef_z=0.0, coef_dev=0.0, stream=None):
    """Allocate the gradients and run moe_backward_saved on forward_train's workspace.
    Returns dict(dx, dWg, dbg, dW1, dW2) and the meta."""
    out = alloc_grads(cfg, x, Wg, W1, W2)
    moe_backward_saved(cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z, coef_dev, out["dx"],
                       out["dWg"], out["dbg"], out["dW1"], out["dW2"], meta, workspace, stream)
    return out, meta


def alloc_workspace(cfg, device="cuda"):
    import torch
    return torch.empty(max(1, moe_workspace_size(cfg)), dtype=torch.uint8, device=device)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def moe_forward(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta, workspace, stream=None):
    """C ABI moe_forward on torch tensors (see include/moe.h for layouts)."""
    c = make_cfg(cfg)
    m = meta.as_struct()
    rc = load_library().moe_forward(
        ctypes.byref(c), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(W2), _ptr(u), _ptr(y),
        _ptr(aux_loss), ctypes.byref(m), _ptr(workspace), workspace.numel(), _stream(stream))
    if rc:
        raise MoeError(rc, "moe_forward")


def moe_forward_noalloc(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta, stream=None):
    """C ABI moe_forward_noalloc (moe_forward on the library's static per-GPU scratch)."""
    c = make_cfg(cfg)
    m = meta.as_struct()
    rc = load_library().moe_forward_noalloc(
        ctypes.byref(c), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(W2), _ptr(u), _ptr(y),
        _ptr(aux_loss), ctypes.byref(m), _stream(stream))
    if rc:
        raise MoeError(rc, "moe_forward_noalloc")


def moe_forward_timed(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta, workspace, events,
                      stream=None):
    """moe_forward recording MOE_N_EVENTS torch.cuda.Event objects at stage boundaries."""
    c = make_cfg(cfg)
    m = meta.as_struct()
    arr = (ctypes.c_void_p * MOE_N_EVENTS)(*[ev.cuda_event for ev in events])
    rc = load_library().moe_forward_timed(
        ctypes.byref(c), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(W2), _ptr(u), _ptr(y),
        _ptr(aux_loss), ctypes.byref(m), _ptr(workspace), workspace.numel(), _stream(stream),
        arr)
    if rc:
        raise MoeError(rc, "moe_forward_timed")


def moe_route(cfg, logits, u, meta, aux_loss, workspace, stream=None):
    """C ABI moe_route: routing, positions, rows and aux from given fp32 logits."""
    c = make_cfg(cfg)
    m = meta.as_struct()
    rc = load_library().moe_route(ctypes.byref(c), _ptr(logits), _ptr(u), ctypes.byref(m),
                                  _ptr(aux_loss), _ptr(workspace), workspace.numel(),
                                  _stream(stream))
    if rc:
        raise MoeError(rc, "moe_route")


def torch_dtype(cfg):
    import torch
    return torch.bfloat16 if cfg["dtype"] == 1 else torch.float32


def forward(cfg, x, Wg, W1, W2, bg=None, u=None, workspace=None, meta=None, y=None,
            stream=None):
    """Allocate outputs (torch.empty) and run moe_forward.  Returns (y, aux_loss, meta)."""
    import torch
    dt = torch_dtype(cfg)
    for name, t in (("x", x), ("Wg", Wg), ("W1", W1), ("W2", W2)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor on the GPU")
    dev = x.device
    meta = alloc_meta(cfg, dev) if meta is None else meta
    y = torch.empty_like(x) if y is None else y
    aux = torch.empty((4,), dtype=torch.float32, device=dev)
    workspace = alloc_workspace(cfg, dev) if workspace is None else workspace
    moe_forward(cfg, x, Wg, bg, W1, W2, u, y, aux, meta, workspace, stream)
    return y, aux[:1], meta
