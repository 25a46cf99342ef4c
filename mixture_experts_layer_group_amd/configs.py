"""The MoE layer workloads used by the parity tests and the benchmark.

Each workload is a plain dict of integers and flags.  The field names are the
ones of the C struct ``moe_cfg`` (include/moe.h) plus the two input-recipe knobs
``zipf_s`` (router offset skew) and ``seed``.

Capacities are stored as the integers the workloads are defined with.  For the
GShard-style layers they equal 2N/(G*E) per group, the fractional capacity of
"GShard: Scaling Giant Models with Conditional Computation and Automatic
Sharding" (section "Top-2 gating 的四个机制 / Local group dispatching").
"""

ACT_RELU, ACT_GELU, ACT_SWIGLU = 0, 1, 2
NORM_NONE, NORM_SUM, NORM_P = 0, 1, 2
DTYPE_F32, DTYPE_BF16 = 0, 1


def _cfg(name, *, n_tokens, n_groups, d_model, d_ff, n_experts, top_k, capacity,
         act, gate_norm, dtype, n_shared=0, random_routing=0, residual=1,
         norm_p=1.0, expert_groups=1, topk_groups=1, zipf_s=0.0, seed=0, desc=""):
    return dict(name=name, n_tokens=n_tokens, n_groups=n_groups, d_model=d_model,
                d_ff=d_ff, n_experts=n_experts, n_shared=n_shared, top_k=top_k,
                capacity=capacity, act=act, gate_norm=gate_norm,
                random_routing=random_routing, residual=residual, dtype=dtype,
                norm_p=norm_p, expert_groups=expert_groups, topk_groups=topk_groups,
                zipf_s=zipf_s, seed=seed, desc=desc)


# The five reference workloads.
WORKLOADS = {
    "tiny_fp32": _cfg(
        "tiny_fp32", n_tokens=256, n_groups=1, d_model=64, d_ff=128, n_experts=4,
        top_k=2, capacity=128, act=ACT_RELU, gate_norm=NORM_SUM, dtype=DTYPE_F32,
        desc="tiny fp32 layer: S=256, M=64, FFN 64->128->64 ReLU, E=4, top-2, C=2S/E=128"),
    "gshard_bf16": _cfg(
        "gshard_bf16", n_tokens=16384, n_groups=8, d_model=1024, d_ff=4096,
        n_experts=64, top_k=2, capacity=64, act=ACT_RELU, gate_norm=NORM_SUM,
        dtype=DTYPE_BF16, random_routing=1,
        desc="GShard-style bf16 layer: G=8 x S=2048, M=1024, FFN 1024->4096->1024 ReLU, "
             "E=64, top-2, C=2S/E=64 per group, random 2nd-expert routing"),
    "switch_bf16": _cfg(
        "switch_bf16", n_tokens=32768, n_groups=1, d_model=768, d_ff=3072,
        n_experts=128, top_k=1, capacity=320, act=ACT_GELU, gate_norm=NORM_NONE,
        dtype=DTYPE_BF16, zipf_s=1.1,
        desc="Switch-style top-1 bf16: 32768 tokens, M=768, FFN 768->3072->768 GELU, "
             "E=128, C=1.25*N/E=320, Zipf(1.1) router offsets"),
    "large_expert_bf16": _cfg(
        "large_expert_bf16", n_tokens=16384, n_groups=1, d_model=4096, d_ff=14336,
        n_experts=8, top_k=2, capacity=16384, act=ACT_GELU, gate_norm=NORM_SUM,
        dtype=DTYPE_BF16,
        desc="large-expert top-2 bf16, dropless (C=N): 16384 tokens, M=4096, "
             "FFN 4096->14336->4096 GELU, E=8"),
    "shared_routed_bf16": _cfg(
        "shared_routed_bf16", n_tokens=32768, n_groups=1, d_model=2048, d_ff=1408,
        n_experts=64, n_shared=2, top_k=6, capacity=4608, act=ACT_GELU,
        gate_norm=NORM_SUM, dtype=DTYPE_BF16, zipf_s=1.2,
        desc="shared+routed bf16: 32768 tokens, M=2048, 2 shared + 64 routed experts "
             "2048->1408->2048 GELU, top-6, C=1.5*6N/64=4608, Zipf(1.2) offsets"),
    # The gated-expert form ([Lec16] "DeepSeek V3 MoE (670B)": SwiGLU experts) on the
    # shared+routed layer above.
    "shared_routed_swiglu_bf16": _cfg(
        "shared_routed_swiglu_bf16", n_tokens=32768, n_groups=1, d_model=2048, d_ff=1408,
        n_experts=64, n_shared=2, top_k=6, capacity=4608, act=ACT_SWIGLU,
        gate_norm=NORM_SUM, dtype=DTYPE_BF16, zipf_s=1.2,
        desc="shared+routed SwiGLU bf16: 32768 tokens, M=2048, 2 shared + 64 routed experts "
             "(Swish(x W1) * x W2) W3 with H=1408, top-6, C=4608, Zipf(1.2) offsets"),
    # Fine-grained experts with group-limited routing, after [Lec16] "DeepSeek V3 MoE
    # (670B)": 256 routed experts in 8 groups of which each token may use 4, 8 active, one
    # shared expert, SwiGLU experts; hidden sizes scaled to M=2048, H=512.
    "fine_grained_grouped_bf16": _cfg(
        "fine_grained_grouped_bf16", n_tokens=16384, n_groups=1, d_model=2048, d_ff=512,
        n_experts=256, n_shared=1, top_k=8, capacity=640, act=ACT_SWIGLU,
        gate_norm=NORM_SUM, expert_groups=8, topk_groups=4, dtype=DTYPE_BF16,
        desc="fine-grained grouped SwiGLU bf16: 16384 tokens, M=2048, 256 routed experts "
             "(H=512) in 8 groups, 4 groups and 8 experts per token, 1 shared expert, "
             "C=1.25*8N/256=640"),
}

# The headline workload of the benchmark (the largest reference layer).
BENCH_WORKLOAD = "large_expert_bf16"

# Small layers the CPU oracle finishes in well under a second that still span several
# GEMM tiles, ragged expert tails, several groups and every gating flag.
SMALL = {
    "small_top2_rr": _cfg(
        "small_top2_rr", n_tokens=1536, n_groups=3, d_model=256, d_ff=384,
        n_experts=8, top_k=2, capacity=96, act=ACT_RELU, gate_norm=NORM_SUM,
        dtype=DTYPE_BF16, random_routing=1, seed=11),
    "small_top1_zipf": _cfg(
        "small_top1_zipf", n_tokens=1000, n_groups=1, d_model=384, d_ff=256,
        n_experts=16, top_k=1, capacity=70, act=ACT_GELU, gate_norm=NORM_NONE,
        dtype=DTYPE_BF16, zipf_s=1.1, seed=12),
    "small_shared_top3": _cfg(
        "small_shared_top3", n_tokens=700, n_groups=1, d_model=256, d_ff=640,
        n_experts=12, n_shared=2, top_k=3, capacity=200, act=ACT_GELU,
        gate_norm=NORM_SUM, dtype=DTYPE_BF16, zipf_s=1.2, seed=13),
    "small_fp32_groups": _cfg(
        "small_fp32_groups", n_tokens=600, n_groups=4, d_model=128, d_ff=192,
        n_experts=6, top_k=2, capacity=30, act=ACT_GELU, gate_norm=NORM_SUM,
        dtype=DTYPE_F32, random_routing=1, seed=14),
    "small_bare_dropless": _cfg(
        "small_bare_dropless", n_tokens=520, n_groups=2, d_model=128, d_ff=256,
        n_experts=5, top_k=2, capacity=260, act=ACT_RELU, gate_norm=NORM_SUM,
        dtype=DTYPE_BF16, residual=0, seed=15),
    "small_swiglu_shared": _cfg(
        "small_swiglu_shared", n_tokens=1200, n_groups=2, d_model=256, d_ff=384,
        n_experts=8, n_shared=1, top_k=2, capacity=140, act=ACT_SWIGLU,
        gate_norm=NORM_SUM, dtype=DTYPE_BF16, zipf_s=0.8, seed=16),
    "small_swiglu_fp32": _cfg(
        "small_swiglu_fp32", n_tokens=500, n_groups=1, d_model=128, d_ff=192,
        n_experts=6, n_shared=2, top_k=3, capacity=220, act=ACT_SWIGLU,
        gate_norm=NORM_SUM, dtype=DTYPE_F32, seed=17),
    "small_pnorm_top4": _cfg(
        "small_pnorm_top4", n_tokens=896, n_groups=2, d_model=256, d_ff=256,
        n_experts=16, top_k=4, capacity=140, act=ACT_GELU, gate_norm=NORM_P, norm_p=2.0,
        dtype=DTYPE_BF16, zipf_s=0.5, seed=18),
    "small_grouped_top4": _cfg(
        "small_grouped_top4", n_tokens=1024, n_groups=2, d_model=256, d_ff=256,
        n_experts=32, top_k=4, capacity=96, act=ACT_SWIGLU, gate_norm=NORM_SUM,
        expert_groups=8, topk_groups=3, dtype=DTYPE_BF16, zipf_s=0.3, seed=20),
    "small_pnorm_half_fp32": _cfg(
        "small_pnorm_half_fp32", n_tokens=384, n_groups=3, d_model=64, d_ff=128,
        n_experts=7, top_k=3, capacity=40, act=ACT_RELU, gate_norm=NORM_P, norm_p=0.5,
        dtype=DTYPE_F32, seed=19),
}

ALL = {**WORKLOADS, **SMALL}

CFG_FIELDS = ("n_tokens", "n_groups", "d_model", "d_ff", "n_experts", "n_shared",
              "top_k", "capacity", "act", "gate_norm", "random_routing", "residual",
              "dtype", "norm_p", "expert_groups", "topk_groups")


def with_overrides(cfg, **kw):
    """Copy of a workload dict with some fields replaced."""
    out = dict(cfg)
    out.update(kw)
    return out
