/*
 * moe.h -- C ABI of the single-GPU mixture-of-experts layer forward pass (gfx950).
 *
 * One call runs the whole layer on one HIP stream:
 *   router GEMM + softmax + top-k gating, per-group expert capacity with overflow drop,
 *   optional random routing of the 2nd expert, dispatch into a compact expert-major
 *   buffer, the two-layer FFN of every expert, and the gate-weighted combine back to
 *   token order (with the residual), plus the auxiliary load-balancing loss.
 *
 * Sources, cited by page title and section:
 *   [GShard]     "GShard: Scaling Giant Models with Conditional Computation and Automatic
 *                Sharding" (reading notes)
 *   [MegaBlocks] "04 · 路由、负载均衡与专家并行" (MegaBlocks router / parallelism chapter)
 *   [Lec16]      "Lec16 Systems for MoE Models" (CMU 11-868 notes)
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major, caller-owned DEVICE memory, 16-byte aligned.  T is
 *     the layer dtype: fp32 (cfg.dtype = MOE_DTYPE_F32) or bf16 (MOE_DTYPE_BF16, passed
 *     as raw 16-bit words).
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is enqueued
 *     asynchronously on it; outputs are valid once the stream has been synchronised.
 *   - The library allocates no device memory and keeps no pointer after returning; calls
 *     with distinct workspaces may run concurrently.  Its only state: moe_forward_noalloc's
 *     static scratch array (one per GPU, see there), and the two side streams of the
 *     backward calls (per GPU, see moe_backward).
 *   - Return value: MOE_OK (0) or a negative MOE_E* code.  All argument checks run on the
 *     host before anything is enqueued; a call that fails them enqueues nothing and writes
 *     nothing.  MOE_EHIP reports a launch error (hipGetLastError) after enqueueing.
 *   - Results are bitwise deterministic for identical inputs (no floating-point atomics).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 2: gated (SwiGLU) experts; 3: p-norm gates, router z-loss; 4: group-limited routing,
 * device-level balance loss; 5: backward pass; 6: moe_forward_noalloc */
#define MOE_ABI_VERSION 7

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* bad cfg, NULL required pointer, pointer not 16-byte aligned */
  MOE_EWORKSPACE = -2,    /* workspace_bytes < moe_workspace_size(cfg) */
  MOE_EUNSUPPORTED = -3,  /* valid cfg outside the kernels' shape constraints */
  MOE_EHIP = -4,          /* a HIP launch failed */
  MOE_ESCRATCH = -5       /* moe_forward_noalloc: the layer needs more workspace than
                             MOE_NOALLOC_SCRATCH_BYTES */
};

/* GELU: exact erf form.  SWIGLU: the gated expert (Swish(x W1) * (x W2)) W3 of [Lec16]
 * "DeepSeek V3 MoE (670B)", Swish(z) = z sigmoid(z); weight layout at moe_forward. */
enum moe_act { MOE_ACT_RELU = 0, MOE_ACT_GELU = 1, MOE_ACT_SWIGLU = 2 };
enum moe_gate_norm { MOE_NORM_NONE = 0, MOE_NORM_SUM = 1, MOE_NORM_P = 2 };
enum moe_dtype { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };

/*
 * Layer configuration (plain old data, all int32).
 *   n_tokens       N >= 0 tokens, split into n_groups contiguous groups of S = N/G tokens
 *                  that route independently ([GShard] "Top-2 gating 的四个机制 / Local group
 *                  dispatching"); N % G == 0, G >= 1.
 *   d_model        M, d_ff H: every expert is act(x W1^T) W2^T, M -> H -> M, no biases
 *                  ([GShard] "MoE Transformer"); with MOE_ACT_SWIGLU it is
 *                  (Swish(x G^T) * (x U^T)) W2^T, G and U the two H-row halves of W1.
 *   n_experts      E routed experts, 1 <= E <= 256.
 *   n_shared       Es >= 0 always-on experts added with weight 1 to every token
 *                  ([Lec16] "共享专家 vs. 路由专家"); they take no capacity and are not in aux.
 *   top_k          1 <= k <= min(E, 8): experts selected per token by the k largest logits,
 *                  descending, ties to the lower expert index.
 *   capacity       C >= 1 slots per (group, expert) ([GShard] "Expert capacity"); C >= S
 *                  means nothing is ever dropped.
 *   act            enum moe_act.
 *   gate_norm      MOE_NORM_SUM: w_j = p_j / sum of the k selected p (softmax over the
 *                  selected logits); MOE_NORM_NONE: w_j = p_j, the full softmax probability;
 *                  MOE_NORM_P: w_j = p_j / (sum_i p_i^P)^(1/P) over the k selected, P =
 *                  norm_p ([MegaBlocks] section 2, optional p-norm of the top-k weights).
 *   random_routing 1: keep the 2nd slot iff u[n] < 2 p2/(p1+p2) ([GShard] "Random routing");
 *                  needs top_k == 2 and a non-NULL u.
 *   residual       1: y = x + layer(x) (a fully dropped token gets y = x exactly);
 *                  0: y = layer(x) (a fully dropped token gets 0).
 *   dtype          enum moe_dtype.
 *   norm_p         P of MOE_NORM_P: finite and > 0 (MOE_EINVAL otherwise); ignored for the
 *                  other gate_norm values.
 *   expert_groups  D, 1 <= D <= 32, E % D == 0: the experts form D contiguous groups of
 *                  E/D ([Lec16] "DeepSeek V3 MoE (670B)": expert groups / limited groups).
 *   topk_groups    1 <= topk_groups <= D: each token keeps the topk_groups groups whose best
 *                  logit is largest (ties to the lower group index) and takes its top-k
 *                  among their experts; needs k <= topk_groups * E/D.  D = 1 (with
 *                  topk_groups = 1) is plain top-k.  The groups also define dev_loss.
 * Shape constraints (MOE_EUNSUPPORTED otherwise):
 *   bf16: M % 128 == 0 and H % 128 == 0.   fp32: M % 64 == 0 and H % 64 == 0.
 *   Sizes: x (N*M elements), the compact row buffers (rows * max(M, H)) and the shared
 *   experts' activations (N*E_sh*H) each under 2^31 bytes, because the kernels address
 *   them through 32-bit buffer ranges.  The backward adds the same bound for its
 *   gradient buffers (see moe_backward_workspace_size).
 */
typedef struct moe_cfg {
  int32_t n_tokens;
  int32_t n_groups;
  int32_t d_model;
  int32_t d_ff;
  int32_t n_experts;
  int32_t n_shared;
  int32_t top_k;
  int32_t capacity;
  int32_t act;
  int32_t gate_norm;
  int32_t random_routing;
  int32_t residual;
  int32_t dtype;
  float norm_p;
  int32_t expert_groups;
  int32_t topk_groups;
} moe_cfg;

/*
 * Dispatch metadata: caller-allocated device arrays the layer fills ([MegaBlocks] section 2
 * returns scores, expert weights and top experts; [Lec16] "MoE Kernel 优化" keeps a dense
 * token-to-expert table).  Every pointer but z_loss and dev_loss is required, and every
 * non-NULL one must be 16-byte aligned.
 *   logits    [N, E] fp32   router logits x Wg^T (+ bg)   (moe_forward only; moe_route
 *                           reads its logits from its own argument and ignores this one)
 *   topk_idx  [N, k] int32  selected experts, descending logit, BEFORE capacity / random
 *                           routing
 *   topk_w    [N, k] fp32   combine weight of each slot; 0 where the slot is not kept
 *                           (no renormalisation after drops)
 *   pos       [N, k] int32  position inside the (group, expert) capacity, -1 if not kept
 *   row       [N, k] int32  row in the compact expert-major buffer, -1 if not kept; rows
 *                           are ordered (expert, group, position)
 *   count     [G, E] int32  kept slots per (group, expert), <= C
 *   offset    [E+1]  int32  first row of each expert; offset[E] = R, the kept slots
 *   stats     [4]    int32  {R, dropped slots, fully dropped tokens, random-routing skips}
 *   z_loss    [1]    fp32   router z-loss, the mean over all N tokens of
 *                           logsumexp(logits_n)^2 ([MegaBlocks] section 2), or NULL: not
 *                           computed.  fp32 logsumexp per token, fp64 fixed-order mean.
 *   dev_loss  [1]    fp32   device-level balance loss over the cfg.expert_groups groups
 *                           ([Lec16] "DeepSeek MoE 的负载均衡"): per token group,
 *                           sum_j f_j P_j with f_j the mean over expert group j of
 *                           f_e = E c_e / (k S) and P_j the sum of m_e over it, averaged
 *                           over token groups (fp64); or NULL: not computed.
 */
typedef struct moe_meta {
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* pos;
  int32_t* row;
  int32_t* count;
  int32_t* offset;
  int32_t* stats;
  float* z_loss;
  float* dev_loss;
} moe_meta;

/* Number of stage boundaries recorded by moe_forward_timed. */
#define MOE_N_EVENTS 7

/* ABI version of the loaded library (MOE_ABI_VERSION at build time). */
int moe_abi_version(void);

/* Static, human-readable description of a moe_status code. */
const char* moe_strerror(int code);

/*
 * Device workspace (bytes) that moe_forward / moe_route need for this cfg.  Host only.
 * Errors: MOE_EINVAL (NULL pointer, bad cfg), MOE_EUNSUPPORTED.
 */
int moe_workspace_size(const moe_cfg* cfg, size_t* bytes);

/*
 * Whole layer forward ([GShard] "MoE 系统的重点是 dispatch/combine": scores -> top-k ->
 * capacity/position -> dispatch -> experts -> combine -> residual, on one GPU).
 *   x         [N, M] T
 *   Wg        [E, M] T      row e = expert e's gate vector ([MegaBlocks] section 2)
 *   bg        [E] fp32 or NULL: fixed per-expert router offsets added to the logits
 *   W1        [E+Es, H, M] T   row n of W1[e] feeds hidden unit n; shared experts last.
 *             MOE_ACT_SWIGLU: [E+Es, 2H, M] T, rows 0..H-1 of W1[e] the Swish (gate)
 *             projection (the formula's W1) and rows H..2H-1 the linear (up) one (its W2)
 *   W2        [E+Es, M, H] T   row m of W2[e] produces output feature m (for
 *             MOE_ACT_SWIGLU, the formula's W3)
 *   u         [N] fp32 in [0,1), required iff cfg.random_routing
 *   y         [N, M] T      output (fp32 accumulation, one rounding to T)
 *   aux_loss  device fp32 scalar: mean over groups of E * sum_e m_e c_e / (k S), with m_e
 *             the group's mean softmax probability and c_e its pre-capacity top-k
 *             selections ([GShard] "Auxiliary loss"; [MegaBlocks] "3. 负载均衡损失")
 *   meta      dispatch metadata (above)
 *   workspace device scratch of at least moe_workspace_size(cfg) bytes; its content on
 *             entry is irrelevant and on exit unspecified
 * N == 0 is valid: only count, offset, stats (zeros) and aux_loss (0) are written, and only
 * cfg, meta->count/offset/stats, aux_loss and workspace are required (others may be NULL).
 * Check order: cfg, then aux_loss/workspace (MOE_EINVAL), then workspace_bytes
 * (MOE_EWORKSPACE), then meta and tensor pointers (MOE_EINVAL).
 */
int moe_forward(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                const void* W1, const void* W2, const float* u, void* y, float* aux_loss,
                const moe_meta* meta, void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_forward, recording `events[0..MOE_N_EVENTS-1]` (caller-created hipEvent_t, passed as
 * void*) on `stream` at the stage boundaries: before the router, after the router, after
 * the capacity scan, after the dispatch scatter, after expert GEMM 1, after expert GEMM 2,
 * after the combine.  Same outputs and errors as moe_forward.
 */
int moe_forward_timed(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                      const void* W1, const void* W2, const float* u, void* y,
                      float* aux_loss, const moe_meta* meta, void* workspace,
                      size_t workspace_bytes, void* stream, void* const* events);

/* Size of moe_forward_noalloc's static scratch array on each GPU (64 MiB). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * moe_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The caller passes the inputs and
 * outputs of moe_forward (same meaning, layouts, results and check order) but no workspace:
 * the library uses a static device array of MOE_NOALLOC_SCRATCH_BYTES on each GPU, which it
 * holds from the first use on that GPU until the process ends.  The call allocates nothing
 * and runs the same kernels as moe_forward.
 *   - The current device (hipSetDevice) must be the device of `stream` and of the tensors.
 *   - MOE_ESCRATCH: moe_workspace_size(cfg) > MOE_NOALLOC_SCRATCH_BYTES (checked on the host
 *     right after cfg; nothing is enqueued).  MOE_EHIP: the scratch array's address could not
 *     be obtained on the current device.
 *   - Every call on one GPU shares that GPU's array, and the array keeps the last call's
 *     contents (none of it needs to start cleared).  Calls that overlap on one GPU (two host
 *     threads, or two streams without ordering between them) race on the array and give
 *     undefined results: serialise them, e.g. on one stream.
 */
int moe_forward_noalloc(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                        const void* W1, const void* W2, const float* u, void* y,
                        float* aux_loss, const moe_meta* meta, void* stream);

/*
 * Device workspace (bytes) that moe_backward needs for this cfg (larger than the forward's).
 * Host only.  Errors: MOE_EINVAL, MOE_EUNSUPPORTED.
 */
int moe_backward_workspace_size(const moe_cfg* cfg, size_t* bytes);

/*
 * Backward pass of the layer: gradients of
 *   L = sum_n <dy_n, y_n> + coef_aux * aux_loss + coef_z * z_loss + coef_dev * dev_loss
 * with respect to x, Wg, bg, W1 and W2 (y, aux_loss, z_loss and dev_loss as in moe_forward).
 * Routing decisions (top-k, group limits, random routing, capacity drops) are constants of
 * the pass ([MegaBlocks] "3. 负载均衡损失": the balance loss reaches the router only through
 * the scores); the rest is the chain rule through combine, the expert FFNs ([GShard] "MoE
 * Transformer"; [Lec16] "DeepSeek V3 MoE (670B)" for the gated form), the gate
 * normalisation and the softmax.  The routing and the expert activations are recomputed
 * from the inputs (the results match a moe_forward of the same inputs bit for bit).
 * Streams: the two weight-gradient GEMMs run on two side streams of the current GPU, each
 * forked from `stream` once its inputs are enqueued and joined back into it before the call
 * returns, so every output is ordered on `stream` as usual.  The library creates those
 * streams and four events on the first backward call on a GPU and keeps them until the
 * process ends; backward calls from several host threads take turns while they enqueue, and
 * their side-stream work runs in the order of the calls.
 *   x, Wg, bg, W1, W2, u   as in moe_forward
 *   dy        [N, M] T      upstream gradient of y
 *   coef_*    host floats (finite) weighting the three auxiliary losses
 *   dx        [N, M] T      out
 *   dWg       [E, M] fp32   out
 *   dbg       [E] fp32 or NULL: gradient of the router offsets
 *   dW1, dW2  fp32, the shapes of W1 and W2: out (experts that received no row get zeros)
 *   meta      as in moe_forward: receives the recomputed routing (logits, topk_idx, topk_w,
 *             pos, row, count, offset, stats); z_loss / dev_loss are not written
 *   workspace device scratch of at least moe_backward_workspace_size(cfg) bytes
 * Precision: the bf16 layer keeps the recomputed pre-activations, activations and every
 * intermediate gradient in bf16, accumulates in fp32, and writes the weight gradients in
 * fp32 (each the sum over its rows in one fixed order: bitwise deterministic).
 * N == 0: the weight gradients are zeroed; meta count/offset/stats are zeroed.
 * Check order: cfg, workspace (MOE_EINVAL), workspace_bytes (MOE_EWORKSPACE), weight-gradient
 * pointers and coefficients, then meta and tensor pointers (MOE_EINVAL).
 */
int moe_backward(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                 const void* W1, const void* W2, const float* u, const void* dy, float coef_aux,
                 float coef_z, float coef_dev, void* dx, float* dWg, float* dbg, float* dW1,
                 float* dW2, const moe_meta* meta, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * Training forward: moe_forward run in a moe_backward workspace that keeps, for
 * moe_backward_saved, the expert activations h and (GELU and SwiGLU layers) their
 * pre-activations, instead of leaving the backward to recompute expert GEMM 1.  This is the
 * other side of the trade-off in [GShard] "Memory 与 Communication" (per-device memory):
 * the activations the backward needs are kept while they fit, and rematerialised only when
 * they do not (moe_backward).
 *   arguments as in moe_forward; y, aux_loss and meta are written exactly as moe_forward
 *   writes them (bit for bit)
 *   workspace device scratch of at least moe_backward_workspace_size(cfg) bytes, owned by
 *             the library from this call until the matching moe_backward_saved call
 * Check order: cfg, workspace (MOE_EINVAL), workspace_bytes against
 * moe_backward_workspace_size (MOE_EWORKSPACE), then as moe_forward.
 */
int moe_forward_train(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                      const void* W1, const void* W2, const float* u, void* y, float* aux_loss,
                      const moe_meta* meta, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * moe_backward that takes h and the pre-activations from the workspace of the preceding
 * moe_forward_train call rather than recomputing expert GEMM 1.  Arguments, outputs, errors
 * and check order as in moe_backward.  The call must use the same cfg, x, Wg, bg, W1, u and
 * workspace as that moe_forward_train call, with nothing else run on the workspace in
 * between (calls on one stream are ordered; across streams the caller orders them).  The
 * routing, and with it every row index, is still recomputed from x and Wg, so a workspace
 * that breaks this contract gives wrong gradients but no access outside the buffers.
 * Results: ReLU layers: every output bit for bit as moe_backward.  GELU and SwiGLU layers:
 * dW1 bit for bit as moe_backward; dW2, and through the combine weights' gradient dx, dWg
 * and dbg, use the forward's h = act(z) rounded once from the fp32 accumulators, where
 * moe_backward recomputes h from the rounded z.
 */
int moe_backward_saved(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                       const void* W1, const void* W2, const float* u, const void* dy,
                       float coef_aux, float coef_z, float coef_dev, void* dx, float* dWg,
                       float* dbg, float* dW1, float* dW2, const moe_meta* meta,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Routing only, from caller-given logits [N, E] fp32: softmax, top-k, gate weights, random
 * routing, capacity positions, dispatch rows and aux ([GShard] "Top-2 gating 的四个机制").
 * Fills meta (except meta->logits, which is not touched and may be NULL) and aux_loss.
 * bg is NOT added here: the logits are taken as final.
 */
int moe_route(const moe_cfg* cfg, const float* logits, const float* u, const moe_meta* meta,
              float* aux_loss, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
