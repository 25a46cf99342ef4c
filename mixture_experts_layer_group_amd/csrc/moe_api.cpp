// Host side of the C ABI in include/moe.h: argument checks, workspace layout, and the
// launch sequence of the MoE layer on one stream.
//
//   moe_router -> moe_gate (capacity scan) -> moe_permute (offsets, positions, scatter)
//   -> expert GEMM 1 (+act) -> expert GEMM 2 -> moe_combine (+aux)
//
// Capacity is static, so every grid size is known on the host; the data-dependent parts
// (kept rows per expert, GEMM tiles) stay on the device and nothing is copied back.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

namespace {

using moe::kRouteTokens;

struct Layout {
  // byte offsets inside the workspace
  size_t buf, h, hsh, osh, active, psum, sel, ahist, abase, ntot, Pg, Cg, tiles, ntiles, zpart,
      tokrow;
  size_t total;
  // sizes
  int64_t S, nbg, Rmax, rows_alloc, max_tiles;
  int esz, BM;
  int group_m;   // m-tile group of the routed GEMM launches
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_cfg(const moe_cfg* c) {
  if (!c) return MOE_EINVAL;
  if (c->n_tokens < 0 || c->n_groups < 1 || c->d_model < 1 || c->d_ff < 1) return MOE_EINVAL;
  if (c->n_tokens % c->n_groups != 0) return MOE_EINVAL;
  if (c->n_experts < 1 || c->n_shared < 0 || c->capacity < 1) return MOE_EINVAL;
  if (c->top_k < 1 || c->top_k > c->n_experts) return MOE_EINVAL;
  if (c->act != MOE_ACT_RELU && c->act != MOE_ACT_GELU && c->act != MOE_ACT_SWIGLU)
    return MOE_EINVAL;
  if (c->gate_norm != MOE_NORM_NONE && c->gate_norm != MOE_NORM_SUM &&
      c->gate_norm != MOE_NORM_P)
    return MOE_EINVAL;
  if (c->gate_norm == MOE_NORM_P && !(c->norm_p > 0.0f && c->norm_p <= FLT_MAX))
    return MOE_EINVAL;  // also rejects NaN and +inf
  if (c->random_routing != 0 && c->random_routing != 1) return MOE_EINVAL;
  if (c->random_routing && c->top_k != 2) return MOE_EINVAL;
  if (c->residual != 0 && c->residual != 1) return MOE_EINVAL;
  if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16) return MOE_EINVAL;
  if (c->expert_groups < 1 || c->n_experts % c->expert_groups != 0) return MOE_EINVAL;
  if (c->topk_groups < 1 || c->topk_groups > c->expert_groups) return MOE_EINVAL;
  if (c->top_k > c->topk_groups * (c->n_experts / c->expert_groups)) return MOE_EINVAL;
  if (c->n_experts > moe::kMaxExperts || c->top_k > moe::kMaxTopK ||
      c->expert_groups > moe::kMaxExpertGroups)
    return MOE_EUNSUPPORTED;
  if (c->dtype == MOE_DTYPE_BF16) {
    if (c->d_model % 128 || c->d_ff % 128) return MOE_EUNSUPPORTED;
  } else {
    if (c->d_model % 64 || c->d_ff % 64) return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

int make_layout(const moe_cfg* c, Layout* L) {
  const int rc = check_cfg(c);
  if (rc) return rc;
  const int64_t N = c->n_tokens, G = c->n_groups, M = c->d_model, H = c->d_ff;
  const int64_t E = c->n_experts, Es = c->n_shared, k = c->top_k, C = c->capacity;
  L->esz = c->dtype == MOE_DTYPE_BF16 ? 2 : 4;
  L->BM = moe::gemm_block_m(c->dtype);
  L->S = N / G;
  L->nbg = (L->S + kRouteTokens - 1) / kRouteTokens;
  L->Rmax = std::min<int64_t>(k * N, G * E * std::min<int64_t>(C, L->S));
  L->rows_alloc = L->Rmax + L->BM;
  L->max_tiles = L->Rmax / L->BM + E + 1;
  L->group_m = moe::gemm_group_m(c->dtype, std::min<int64_t>(N, G * std::min<int64_t>(C, L->S)));
  // 32-bit limits of the kernels: element indices, and the byte range of a buffer resource
  // (GEMM 1 gathers its rows from the whole of x through one resource; h, o and the shared
  // output are addressed from tile bases inside their buffers)
  const int64_t lim = (int64_t{1} << 31) - 1;
  const int64_t eb = L->esz;
  if (N * k > lim || N * std::max<int64_t>(M, E) > lim || N * M * eb > lim ||
      L->rows_alloc * std::max(M, H) * eb > lim || (E + Es) * M * H > lim ||
      N * Es * H * eb > lim || G * k * E * L->nbg > lim)
    return MOE_EUNSUPPORTED;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t esz = static_cast<size_t>(L->esz);
  L->buf = take(static_cast<size_t>(L->rows_alloc) * M * esz);    // dispatched rows, then o
  L->h = take(static_cast<size_t>(L->rows_alloc) * H * esz);
  L->hsh = take(static_cast<size_t>(N) * Es * H * esz);
  L->osh = take(static_cast<size_t>(N) * (Es ? M : 0) * esz);
  L->active = take(static_cast<size_t>(N) * k);
  L->psum = take(static_cast<size_t>(G) * E * L->nbg * 8);
  L->sel = take(static_cast<size_t>(G) * E * L->nbg * 4);
  L->ahist = take(static_cast<size_t>(G) * k * E * L->nbg * 4);
  L->abase = take(static_cast<size_t>(G) * k * E * L->nbg * 4);
  L->ntot = take(static_cast<size_t>(G) * k * E * 4);
  L->Pg = take(static_cast<size_t>(G) * E * 8);
  L->Cg = take(static_cast<size_t>(G) * E * 4);
  L->tiles = take(static_cast<size_t>(L->max_tiles) * sizeof(moe::TileDesc));
  L->ntiles = take(16);
  L->zpart = take(static_cast<size_t>(G) * L->nbg * 8);
  L->tokrow = take(static_cast<size_t>(L->rows_alloc) * 4);
  L->total = off;
  return MOE_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_meta(const moe_meta* m, bool need_logits) {
  if (!m) return MOE_EINVAL;
  const void* ps[] = {m->topk_idx, m->topk_w, m->pos, m->row, m->count, m->offset, m->stats};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return MOE_EINVAL;
  if (need_logits && (!m->logits || !aligned16(m->logits))) return MOE_EINVAL;
  if (m->z_loss && !aligned16(m->z_loss)) return MOE_EINVAL;  // optional outputs
  if (m->dev_loss && !aligned16(m->dev_loss)) return MOE_EINVAL;
  return MOE_OK;
}

// N == 0: only count, offset, stats (and z_loss / dev_loss if requested) are written.
int check_meta_empty(const moe_meta* m) {
  if (!m || !m->count || !m->offset || !m->stats) return MOE_EINVAL;
  if (m->z_loss && !aligned16(m->z_loss)) return MOE_EINVAL;
  if (m->dev_loss && !aligned16(m->dev_loss)) return MOE_EINVAL;
  return MOE_OK;
}

struct Run {
  const moe_cfg* c;
  Layout L;
  char* ws;
  hipStream_t s;
};

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

void record(void* const* ev, int i, hipStream_t s) {
  if (ev && ev[i]) hipEventRecord(static_cast<hipEvent_t>(ev[i]), s);
}

// Router (or routing from given logits) + scan + offsets + positions/scatter.
// copy_rows: also copy the kept token rows into the compact buffer (the backward reads them);
// the forward's GEMM 1 gathers them from x through tok_of_row instead.  The backward also
// passes dy: then dout[row] = w dy[n] for every kept slot and wrow[row] = w.
int run_routing(const Run& r, const void* x, const void* Wg, const float* bg, const float* u,
                const float* logits_in, const moe_meta* m, int bm, void* const* ev,
                bool copy_rows, const void* dy = nullptr, void* dout = nullptr,
                float* wrow = nullptr) {
  const moe_cfg* c = r.c;
  const Layout& L = r.L;
  char* ws = r.ws;
  moe::RouterArgs ra{};
  ra.x = x; ra.Wg = Wg; ra.bg = bg; ra.u = u; ra.logits_in = logits_in;
  ra.logits_out = logits_in ? nullptr : m->logits;
  ra.topk_idx = m->topk_idx; ra.topk_w = m->topk_w;
  ra.active = reinterpret_cast<uint8_t*>(ws + L.active);
  ra.psum = reinterpret_cast<double*>(ws + L.psum);
  ra.sel = reinterpret_cast<int32_t*>(ws + L.sel);
  ra.ahist = reinterpret_cast<int32_t*>(ws + L.ahist);
  ra.zpart = reinterpret_cast<double*>(ws + L.zpart);
  ra.norm_p = c->norm_p;
  ra.n_eg = c->expert_groups; ra.topk_eg = c->topk_groups;
  ra.N = c->n_tokens; ra.G = c->n_groups; ra.S = static_cast<int>(L.S); ra.M = c->d_model;
  ra.E = c->n_experts; ra.k = c->top_k; ra.norm = c->gate_norm; ra.rr = c->random_routing;
  ra.nbg = static_cast<int>(L.nbg); ra.dtype = c->dtype;
  record(ev, 0, r.s);
  int rc = status_of(moe::launch_router(ra, r.s));
  if (rc) return rc;
  record(ev, 1, r.s);

  moe::ScanArgs sa{};
  sa.ahist = ra.ahist; sa.psum = ra.psum; sa.sel = ra.sel;
  sa.abase = reinterpret_cast<int32_t*>(ws + L.abase);
  sa.count = m->count;
  sa.ntot = reinterpret_cast<int32_t*>(ws + L.ntot);
  sa.Pg = reinterpret_cast<double*>(ws + L.Pg);
  sa.Cg = reinterpret_cast<int32_t*>(ws + L.Cg);
  sa.G = c->n_groups; sa.E = c->n_experts; sa.k = c->top_k; sa.C = c->capacity;
  sa.nbg = static_cast<int>(L.nbg);
  sa.stats = m->stats;
  rc = status_of(moe::launch_gate_scan(sa, r.s));
  if (rc) return rc;
  record(ev, 2, r.s);

  moe::PermuteArgs pa{};
  pa.x = copy_rows ? x : nullptr;
  pa.tok_of_row = reinterpret_cast<int32_t*>(ws + L.tokrow);
  pa.topk_idx = m->topk_idx; pa.active = ra.active; pa.abase = sa.abase;
  pa.count = m->count; pa.ntot = sa.ntot; pa.offset = m->offset;
  pa.tiles = reinterpret_cast<moe::TileDesc*>(ws + L.tiles);
  pa.num_tiles = reinterpret_cast<int32_t*>(ws + L.ntiles);
  pa.pos = m->pos; pa.row = m->row; pa.topk_w = m->topk_w;
  pa.stats = m->stats; pa.buf = ws + L.buf;
  pa.dy = copy_rows ? dy : nullptr; pa.dout = dout; pa.w_of_row = wrow;
  pa.N = c->n_tokens; pa.G = c->n_groups; pa.S = static_cast<int>(L.S); pa.M = c->d_model;
  pa.E = c->n_experts; pa.k = c->top_k; pa.C = c->capacity; pa.nbg = static_cast<int>(L.nbg);
  pa.dtype = c->dtype; pa.BM = bm;
  rc = status_of(moe::launch_permute(pa, r.s));
  if (rc) return rc;
  record(ev, 3, r.s);
  return MOE_OK;
}

moe::CombineArgs combine_args(const Run& r, const void* x, void* y, float* aux,
                              const moe_meta* m) {
  const moe_cfg* c = r.c;
  moe::CombineArgs ca{};
  ca.x = x; ca.o = r.ws + r.L.buf; ca.o_sh = c->n_shared ? r.ws + r.L.osh : nullptr;
  ca.row = m->row; ca.topk_w = m->topk_w; ca.y = y;
  ca.Pg = reinterpret_cast<const double*>(r.ws + r.L.Pg);
  ca.Cg = reinterpret_cast<const int32_t*>(r.ws + r.L.Cg);
  ca.aux = aux;
  ca.zpart = reinterpret_cast<const double*>(r.ws + r.L.zpart);
  ca.z_loss = m->z_loss;
  ca.dev_loss = m->dev_loss;
  ca.n_eg = c->expert_groups;
  ca.nblocks = static_cast<int>(c->n_groups * r.L.nbg);
  ca.N = c->n_tokens; ca.M = c->d_model; ca.k = c->top_k; ca.residual = c->residual;
  ca.dtype = c->dtype; ca.G = c->n_groups; ca.E = c->n_experts; ca.S = static_cast<int>(r.L.S);
  return ca;
}

int empty_call(const moe_cfg* c, const moe_meta* m, float* aux, hipStream_t s, void* const* ev) {
  moe::EmptyArgs ea{m->count, m->offset, m->stats, aux, m->z_loss, m->dev_loss,
                    c->n_groups, c->n_experts};
  for (int i = 0; i < MOE_N_EVENTS - 1; ++i) record(ev, i, s);
  const int rc = status_of(moe::launch_empty(ea, s));
  record(ev, MOE_N_EVENTS - 1, s);
  return rc;
}

// Where the training forward keeps GEMM 1's pre-activations (GELU and SwiGLU layers): z1
// [rows, H1] in compact row order and z1sh [N, Es H1].
struct TrainOut {
  void* z1;
  void* z1sh;
};

// Tile order of GEMM 1 (forward, and the backward's recompute): 2 = expert-synchronous when
// there are no shared experts and the weights of min(E, 8) experts exceed 256 MB, else 0.
int esync_gemm1(int64_t E, int64_t Es, int64_t H1, int64_t M, int64_t esz) {
  return !Es && std::min<int64_t>(E, 8) * H1 * M * esz > (int64_t{256} << 20) ? 2 : 0;
}

// check_only: run every host check and return without enqueueing anything.  train: also
// store GEMM 1's pre-activations there (ReLU layers keep h only).
int forward_impl(const moe_cfg* c, const void* x, const void* Wg, const float* bg,
                 const void* W1, const void* W2, const float* u, void* y, float* aux,
                 const moe_meta* m, void* workspace, size_t wbytes, void* stream,
                 void* const* ev, bool check_only = false, const TrainOut* train = nullptr) {
  Run r;
  r.c = c;
  int rc = make_layout(c, &r.L);
  if (rc) return rc;
  if (!aux || !aligned16(aux) || !workspace || !aligned16(workspace)) return MOE_EINVAL;
  if (wbytes < r.L.total) return MOE_EWORKSPACE;
  if (c->n_tokens == 0) {
    // Nothing to route: only the small outputs are written; token pointers may be NULL.
    rc = check_meta_empty(m);
    if (rc || check_only) return rc;
    return empty_call(c, m, aux, static_cast<hipStream_t>(stream), ev);
  }
  rc = check_meta(m, true);
  if (rc) return rc;
  if (c->random_routing && (!u || !aligned16(u))) return MOE_EINVAL;
  if (bg && !aligned16(bg)) return MOE_EINVAL;
  const void* req[] = {x, Wg, W1, W2, y};
  for (const void* p : req)
    if (!p || !aligned16(p)) return MOE_EINVAL;
  if (check_only) return MOE_OK;
  r.ws = static_cast<char*>(workspace);
  r.s = static_cast<hipStream_t>(stream);

  const int64_t M = c->d_model, H = c->d_ff, E = c->n_experts, Es = c->n_shared;
  const int BM = r.L.BM;
  rc = run_routing(r, x, Wg, bg, u, nullptr, m, BM, ev, false);
  if (rc) return rc;

  const Layout& L = r.L;
  char* ws = r.ws;
  const moe::TileDesc* tiles = reinterpret_cast<const moe::TileDesc*>(ws + L.tiles);
  const int32_t* ntiles = reinterpret_cast<const int32_t*>(ws + L.ntiles);
  const int a_rows = static_cast<int>(L.rows_alloc);

  // GEMM 1: h = act(x[tok] . W1_e^T) for every expert, the token rows gathered from x in
  // compact (expert-major) order (+ shared: h_sh = act(x . W1_sh^T)).
  // Gated experts: h = Swish(x . G_e^T) * (x . U_e^T) from W1_e = [G_e; U_e] (2H rows).
  const int64_t H1 = c->act == MOE_ACT_SWIGLU ? 2 * H : H;  // W1 rows per expert
  moe::GemmArgs g1{};
  g1.dtype = c->dtype;
  g1.p0 = moe::GemmProblem{x, M, W1, M, H1 * M, M, 0, ws + L.h, H,
                           static_cast<int>(H), static_cast<int>(M), c->n_tokens, c->act,
                           tiles, ntiles, static_cast<int>(L.max_tiles), 0,
                           static_cast<int>(H)};
  g1.p0.a_gather = reinterpret_cast<const int32_t*>(ws + L.tokrow);
  g1.nprob = 1;
  // Expert-synchronous tile order when the weights of the 8 experts that the XCD ranges run
  // at once (one per XCD) overflow the 256 MB last-level cache; otherwise the XCD ranges read
  // every weight and every gathered row once.
  g1.plain = esync_gemm1(E, Es, H1, M, L.esz);
  if (Es) {
    const char* w1sh = static_cast<const char*>(W1) + E * H1 * M * L.esz;
    g1.p1 = moe::GemmProblem{x, M, w1sh, M, 0, M, 0, ws + L.hsh, Es * H,
                             static_cast<int>(Es * H), static_cast<int>(M), c->n_tokens,
                             c->act, nullptr, nullptr,
                             static_cast<int>((c->n_tokens + BM - 1) / BM), c->n_tokens,
                             static_cast<int>(H)};
    g1.nprob = 2;
  }
  if (train && c->act != MOE_ACT_RELU) {
    g1.p0.zout = train->z1;
    g1.p0.ldz = H1;
    g1.p1.zout = train->z1sh;
    g1.p1.ldz = Es * H1;
  }
  g1.group_m = L.group_m;
  rc = status_of(moe::launch_expert_gemm(g1, r.s));
  if (rc) return rc;
  record(ev, 4, r.s);

  // GEMM 2: o = h . W2_e^T into the dispatch buffer (+ shared: o_sh = h_sh . [W2_sh...]^T).
  moe::GemmArgs g2{};
  g2.dtype = c->dtype;
  g2.p0 = moe::GemmProblem{ws + L.h, H, W2, H, M * H, H, 0, ws + L.buf, M,
                           static_cast<int>(M), static_cast<int>(H), a_rows, moe::kActNone,
                           tiles, ntiles, static_cast<int>(L.max_tiles), 0, 0};
  g2.nprob = 1;
  if (Es) {
    const char* w2sh = static_cast<const char*>(W2) + E * M * H * L.esz;
    g2.p1 = moe::GemmProblem{ws + L.hsh, Es * H, w2sh, H, 0, H, M * H, ws + L.osh, M,
                             static_cast<int>(M), static_cast<int>(Es * H), c->n_tokens,
                             moe::kActNone, nullptr, nullptr,
                             static_cast<int>((c->n_tokens + BM - 1) / BM), c->n_tokens, 0};
    g2.nprob = 2;
  }
  g2.group_m = L.group_m;
  // h larger than the last-level cache (256 MB): plain tile order (see tile_coord)
  g2.plain = !Es && L.Rmax * H * L.esz > (int64_t{256} << 20);
  rc = status_of(moe::launch_expert_gemm(g2, r.s));
  if (rc) return rc;
  record(ev, 5, r.s);

  rc = status_of(moe::launch_combine(combine_args(r, x, y, aux, m), r.s));
  record(ev, 6, r.s);
  return rc;
}

// ---------------------------------------------------------------------------- backward

// The backward's side streams.  The weight gradients of the two expert GEMMs depend only on
// activations the chain has already produced (dW2 on h and dout, dW1 on dz and the dispatched
// rows), not on the dgrad kernels after them, so each runs on a stream of its own beside
// those kernels, from the moment its inputs exist: their fp32 tile stores, which leave the
// MFMA pipes idle, overlap compute-bound work.  Two non-blocking, default-priority streams and
// four timing-free events per device, created on first use and kept until the process ends.
// A backward call holds the mutex while it enqueues, so calls from several host threads do
// not interleave their records.
struct SideStream {
  hipStream_t s[2] = {};
  hipEvent_t ev[4] = {};
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// The current device's side streams (created if needed); the caller holds g_side_mu.
int side_stream(SideStream** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  SideStream& ss = g_side[dev];
  if (!ss.s[0]) {
    SideStream n;
    for (hipStream_t& st : n.s)
      if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return MOE_EHIP;
    for (hipEvent_t& e : n.ev)
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return MOE_EHIP;
    ss = n;
  }
  *out = &ss;
  return MOE_OK;
}

// Fork / join of the side streams: fork(i) makes side stream i wait for what the main stream
// has enqueued so far; the join (at the latest when this object goes out of scope, error
// paths included) makes the main stream wait for everything enqueued on both.
struct SideFork {
  SideStream* ss = nullptr;
  hipStream_t main = nullptr;
  bool open[2] = {false, false};
  int fork(int i) {
    if (hipEventRecord(ss->ev[i], main) != hipSuccess ||
        hipStreamWaitEvent(ss->s[i], ss->ev[i], 0) != hipSuccess)
      return MOE_EHIP;
    open[i] = true;
    return MOE_OK;
  }
  int join() {
    int rc = MOE_OK;
    for (int i = 0; i < 2; ++i) {
      if (!open[i]) continue;
      open[i] = false;
      if (hipEventRecord(ss->ev[2 + i], ss->s[i]) != hipSuccess ||
          hipStreamWaitEvent(main, ss->ev[2 + i], 0) != hipSuccess)
        rc = MOE_EHIP;
    }
    return rc;
  }
  ~SideFork() { join(); }
};

// Workspace of moe_backward: the forward layout (routing buffers, dispatch rows, h, shared h,
// and the shared-output buffer reused for the shared experts' dx), then the backward's own
// regions.  Every GEMM reads its operands in place (weights and activations as K-major
// operands where the contraction runs along their rows), so no transposed copies are kept.
struct BwdLayout {
  Layout F;
  size_t z1, dout, wrow, dwp, dz1, dbuf, z1sh, dz1sh, dl, dw, partb, dlp, dxrt, e2, e1, eh,
      eg, dwgp, shp2, shp1, total;
  int64_t H1, nchunks, Ep, nsplit, ksplit, nshared, kshared, ntn;
};

int make_bwd_layout(const moe_cfg* c, BwdLayout* B) {
  int rc = make_layout(c, &B->F);
  if (rc) return rc;
  const Layout& L = B->F;
  const int64_t N = c->n_tokens, M = c->d_model, H = c->d_ff, E = c->n_experts;
  const int64_t Es = c->n_shared, k = c->top_k;
  const int64_t H1 = c->act == MOE_ACT_SWIGLU ? 2 * H : H;
  B->H1 = H1;
  if (Es > 256) return MOE_EUNSUPPORTED;          // one setup thread per shared expert
  B->nchunks = (N + 255) / 256;
  B->Ep = (E + 63) / 64 * 64;
  // dWg [E, M] contracts over all N tokens but has few output tiles: split the token axis
  // into ranges of a multiple of 128 tokens so that about 256 tiles run, partials in fp32
  {
    const int64_t tiles = ((E + 255) / 256) * ((M + 255) / 256);
    const int64_t Npad = (N + 127) / 128 * 128;
    const int64_t S = std::max<int64_t>(1, std::min<int64_t>((256 + tiles - 1) / tiles, Npad / 128));
    B->ksplit = std::max<int64_t>(128, (Npad / S + 127) / 128 * 128);
    B->nsplit = (N + B->ksplit - 1) / B->ksplit;   // 0 for an empty batch
  }
  // The shared experts' weight gradients contract over all N tokens: split that axis into
  // ranges about as long as a routed expert's kept rows (N k / E), so that their tiles are not
  // a tail of the launch; partials in fp32 (at most 32 ranges)
  {
    const int64_t avg = (N * k + E - 1) / std::max<int64_t>(E, 1);
    B->kshared = std::max<int64_t>(512, (avg + 127) / 128 * 128);
    B->kshared = std::max(B->kshared, (N + 31) / 32);
    B->nshared = Es ? (N + B->kshared - 1) / B->kshared : 0;
  }
  // every operand a GEMM reads through a buffer resource stays under 2 GiB
  const int64_t lim = (int64_t{1} << 31) - 1;
  const int64_t esz = L.esz, ra = L.rows_alloc;
  if (ra * H1 * esz > lim || ra * M * esz > lim || (E + Es) * H1 * M * esz > lim ||
      N * Es * H1 * esz > lim || N * std::max(M, B->Ep) * esz > lim || N * Es * H * esz > lim)
    return MOE_EUNSUPPORTED;
  size_t off = L.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t es = static_cast<size_t>(esz), rs = static_cast<size_t>(ra);
  const bool relu = c->act == MOE_ACT_RELU;   // ReLU keeps h instead of z1
  B->z1 = take(relu ? 0 : rs * H1 * es);
  B->dout = take(rs * M * es);
  B->ntn = (H + moe::gemm_block_n(c->dtype, moe::kActNone) - 1) / moe::gemm_block_n(c->dtype, moe::kActNone);
  B->wrow = take(rs * 4);
  B->dwp = take(rs * static_cast<size_t>(B->ntn) * 4);
  B->dz1 = take(rs * H1 * es);
  B->dbuf = take(rs * M * es);
  B->z1sh = take(relu ? 0 : static_cast<size_t>(N * Es * H1) * es);
  B->dz1sh = take(static_cast<size_t>(N * Es * H1) * es);
  B->dl = take(static_cast<size_t>(N * E) * 4);
  B->dw = take(static_cast<size_t>(N * k) * 4);
  B->partb = take(static_cast<size_t>(B->nchunks * E) * 4);
  B->dlp = take(static_cast<size_t>(N * B->Ep) * es);
  B->dxrt = take(static_cast<size_t>(N * M) * es);
  B->e2 = take(static_cast<size_t>(E + Es * B->nshared) * sizeof(moe::BatchEntry));
  B->e1 = take(static_cast<size_t>(E + Es * B->nshared) * sizeof(moe::BatchEntry));
  B->eh = take(static_cast<size_t>(Es) * sizeof(moe::BatchEntry));
  B->eg = take(static_cast<size_t>(B->nsplit) * sizeof(moe::BatchEntry));
  B->dwgp = take(static_cast<size_t>(B->nsplit * E * M) * 4);
  B->shp2 = take(static_cast<size_t>(Es * B->nshared * M * H) * 4);
  B->shp1 = take(static_cast<size_t>(Es * B->nshared * H1 * M) * 4);
  B->total = off;
  return MOE_OK;
}

moe::GemmProblem routed_problem(const void* A, int64_t lda, const void* Bm, int64_t ldb,
                                int64_t bstride, void* C, int64_t ldc, int N, int K,
                                int a_rows, const Layout& L, const moe::TileDesc* tiles,
                                const int32_t* ntiles) {
  moe::GemmProblem p{};
  p.A = A; p.lda = lda; p.B = Bm; p.ldb = ldb; p.b_stride = bstride; p.kseg = K;
  p.C = C; p.ldc = ldc; p.N = N; p.K = K; p.a_rows = a_rows; p.act = moe::kActNone;
  p.tiles = tiles; p.num_tiles = ntiles; p.max_tiles = static_cast<int>(L.max_tiles);
  return p;
}

moe::GemmProblem dense_problem(const void* A, int64_t lda, const void* Bm, int64_t ldb,
                               void* C, int64_t ldc, int N, int K, int rows, int BM) {
  moe::GemmProblem p{};
  p.A = A; p.lda = lda; p.B = Bm; p.ldb = ldb; p.kseg = K;
  p.C = C; p.ldc = ldc; p.N = N; p.K = K; p.a_rows = rows; p.act = moe::kActNone;
  p.max_tiles = (rows + BM - 1) / BM; p.dense_rows = rows;
  return p;
}

// Batched problem: entry i multiplies rows [0, rows) of A + a_off_i by B + b_off_i over its own
// K into C + c_off_i (entries built on the device).
moe::GemmProblem batched_problem(const void* A, int64_t lda, const void* Bm, int64_t ldb,
                                 void* C, int64_t ldc, int N, int rows, int entries, int BM,
                                 const moe::BatchEntry* batch, bool out_f32) {
  moe::GemmProblem p{};
  p.A = A; p.lda = lda; p.B = Bm; p.ldb = ldb; p.kseg = int64_t{1} << 30;  // no K segments
  p.C = C; p.ldc = ldc; p.N = N; p.K = 0; p.a_rows = rows; p.act = moe::kActNone;
  p.max_tiles = entries * ((rows + BM - 1) / BM); p.dense_rows = rows;
  p.batch = batch; p.out_f32 = out_f32 ? 1 : 0;
  return p;
}

// saved: h (and for GELU / SwiGLU z1) are the training forward's, already in the workspace,
// and GEMM 1 is not recomputed.  The routing is recomputed either way.
int backward_impl(const moe_cfg* c, const void* x, const void* Wg, const float* bg,
                  const void* W1, const void* W2, const float* u, const void* dy,
                  float coef_aux, float coef_z, float coef_dev, void* dx, float* dWg,
                  float* dbg, float* dW1, float* dW2, const moe_meta* m, void* workspace,
                  size_t wbytes, void* stream, bool saved = false) {
  BwdLayout B;
  int rc = make_bwd_layout(c, &B);
  if (rc) return rc;
  if (!workspace || !aligned16(workspace)) return MOE_EINVAL;
  if (wbytes < B.total) return MOE_EWORKSPACE;
  const float* req_f[] = {dWg, dW1, dW2};
  for (const float* p : req_f)
    if (!p || !aligned16(p)) return MOE_EINVAL;
  if (dbg && !aligned16(dbg)) return MOE_EINVAL;
  if (!std::isfinite(coef_aux) || !std::isfinite(coef_z) || !std::isfinite(coef_dev))
    return MOE_EINVAL;
  const int64_t N = c->n_tokens, M = c->d_model, H = c->d_ff, E = c->n_experts;
  const int64_t Es = c->n_shared, k = c->top_k, H1 = B.H1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) {  // no tokens: every gradient is zero
    rc = check_meta_empty(m);
    if (rc) return rc;
    rc = status_of(moe::launch_zero(dWg, E * M, s));
    if (!rc) rc = status_of(moe::launch_zero(dW1, (E + Es) * H1 * M, s));
    if (!rc) rc = status_of(moe::launch_zero(dW2, (E + Es) * M * H, s));
    if (!rc && dbg) rc = status_of(moe::launch_zero(dbg, E, s));
    if (rc) return rc;
    moe::EmptyArgs ea{m->count, m->offset, m->stats, nullptr, m->z_loss, m->dev_loss,
                      c->n_groups, c->n_experts};
    return status_of(moe::launch_empty(ea, s));
  }
  rc = check_meta(m, true);
  if (rc) return rc;
  if (c->random_routing && (!u || !aligned16(u))) return MOE_EINVAL;
  if (bg && !aligned16(bg)) return MOE_EINVAL;
  const void* req[] = {x, Wg, W1, W2, dy, dx};
  for (const void* p : req)
    if (!p || !aligned16(p)) return MOE_EINVAL;

  std::lock_guard<std::mutex> lock(g_side_mu);
  SideFork side;   // joined before the lock is released
  rc = side_stream(&side.ss);
  if (rc) return rc;
  side.main = s;
  const hipStream_t s2 = side.ss->s[0], s3 = side.ss->s[1];

  Run r;
  r.c = c;
  r.L = B.F;
  r.ws = static_cast<char*>(workspace);
  r.s = s;
  const Layout& L = B.F;
  char* ws = r.ws;
  const int BM = L.BM, dt = c->dtype;
  const size_t esz = static_cast<size_t>(L.esz);
  // 1. routing again (deterministic: the forward's routing), rows dispatched into buf
  float* wrow = reinterpret_cast<float*>(ws + B.wrow);
  rc = run_routing(r, x, Wg, bg, u, nullptr, m, BM, nullptr, true, dy, ws + B.dout, wrow);
  if (rc) return rc;
  const moe::TileDesc* tiles = reinterpret_cast<const moe::TileDesc*>(ws + L.tiles);
  const int32_t* ntiles = reinterpret_cast<const int32_t*>(ws + L.ntiles);
  const int32_t* Rdev = m->offset + E;  // kept rows
  const int a_rows = static_cast<int>(L.rows_alloc);
  const char* W1c = static_cast<const char*>(W1);
  const char* W2c = static_cast<const char*>(W2);
  auto gemm = [&](const moe::GemmProblem& p0, const moe::GemmProblem* p1,
                  hipStream_t st = nullptr, int plain = 0) {
    moe::GemmArgs g{};
    g.dtype = dt; g.p0 = p0; g.nprob = 1; g.plain = plain;
    if (p0.tiles) g.group_m = L.group_m;   // routed launches
    if (p1) { g.p1 = *p1; g.nprob = 2; }
    return status_of(moe::launch_expert_gemm(g, st ? st : s));
  };
  const int nsh = static_cast<int>(Es * B.nshared);
  float* shp2 = reinterpret_cast<float*>(ws + B.shp2);
  float* shp1 = reinterpret_cast<float*>(ws + B.shp1);
  // batched GEMM entries of the steps below, from the expert offsets
  moe::BwdSetupArgs sa{};
  sa.offset = m->offset;
  sa.dw2 = reinterpret_cast<moe::BatchEntry*>(ws + B.e2);
  sa.dw1 = reinterpret_cast<moe::BatchEntry*>(ws + B.e1);
  sa.dhsh = reinterpret_cast<moe::BatchEntry*>(ws + B.eh);
  sa.dwg = reinterpret_cast<moe::BatchEntry*>(ws + B.eg);
  sa.E = static_cast<int>(E); sa.Es = static_cast<int>(Es); sa.M = static_cast<int>(M);
  sa.H = static_cast<int>(H); sa.H1 = static_cast<int>(H1); sa.N = static_cast<int>(N);
  sa.Ep = static_cast<int>(B.Ep);
  sa.nsplit = static_cast<int>(B.nsplit);
  sa.ksplit = static_cast<int>(B.ksplit);
  sa.nshared = static_cast<int>(B.nshared);
  sa.kshared = static_cast<int>(B.kshared);
  rc = status_of(moe::launch_bwd_setup(sa, s));
  if (rc) return rc;
  // 2. h = act(z1) with z1 = buf W1_e^T (routed) and x W1_sh^T (shared), and z1 beside it.
  //    ReLU needs no z1: ReLU'(z1) is 1 exactly where h > 0, so GEMM 1 writes h as in the
  //    forward.
  const bool relu = c->act == MOE_ACT_RELU;
  // the forward GEMM 1's tile order (weights larger than the last-level cache)
  const int plain1 = esync_gemm1(E, Es, H1, M, L.esz);
  if (saved) {
    // kept by the training forward
  } else if (relu) {
    auto p0 = routed_problem(ws + L.buf, M, W1, M, H1 * M, ws + L.h, H, static_cast<int>(H),
                             static_cast<int>(M), a_rows, L, tiles, ntiles);
    auto p1 = dense_problem(x, M, W1c + E * H1 * M * esz, M, ws + L.hsh, Es * H,
                            static_cast<int>(Es * H), static_cast<int>(M),
                            static_cast<int>(N), BM);
    p0.act = p1.act = moe::kActRelu;
    rc = gemm(p0, Es ? &p1 : nullptr, nullptr, plain1);
    if (rc) return rc;
  } else {
    // the training forward's GEMM 1: h from the fp32 accumulators through the forward's own
    // activation epilogue, and the pre-activations z1 beside it, so that the recomputed h is
    // the forward's bit for bit (an activation applied to the rounded z1 afterwards would not
    // be)
    auto p0 = routed_problem(ws + L.buf, M, W1, M, H1 * M, ws + L.h, H, static_cast<int>(H),
                             static_cast<int>(M), a_rows, L, tiles, ntiles);
    auto p1 = dense_problem(x, M, W1c + E * H1 * M * esz, M, ws + L.hsh, Es * H,
                            static_cast<int>(Es * H), static_cast<int>(M),
                            static_cast<int>(N), BM);
    p0.act = p1.act = c->act;
    p0.glu_h = p1.glu_h = static_cast<int>(H);
    p0.zout = ws + B.z1;
    p0.ldz = H1;
    p1.zout = ws + B.z1sh;
    p1.ldz = Es * H1;
    rc = gemm(p0, Es ? &p1 : nullptr, nullptr, plain1);
    if (rc) return rc;
  }
  // 6a. (first side stream, beside steps 3-5) dW2_e [M, H] = dout_e^T h_e; shared q: dy^T hsh_q
  //     over token ranges into fp32 partials, summed in range order.  Weight gradients are
  //     fp32 batched GEMMs over the experts with K = the expert's kept rows (shared experts:
  //     all tokens), every operand read in place as a K-major operand.
  {
    if ((rc = side.fork(0))) return rc;
    auto q0 = batched_problem(ws + B.dout, M, ws + L.h, H, dW2, H, static_cast<int>(H),
                              static_cast<int>(M), static_cast<int>(E), BM, sa.dw2, true);
    auto q1 = batched_problem(dy, M, ws + L.hsh, Es * H, shp2, H, static_cast<int>(H),
                              static_cast<int>(M), nsh, BM, sa.dw2 + E, true);
    q0.a_kmajor = q0.b_kmajor = q1.a_kmajor = q1.b_kmajor = 1;
    if ((rc = gemm(q0, Es ? &q1 : nullptr, s2))) return rc;
    for (int64_t q = 0; q < Es; ++q)
      if ((rc = status_of(moe::launch_split_reduce(shp2 + q * B.nshared * M * H,
                                                   dW2 + (E + q) * M * H, M * H,
                                                   static_cast<int>(B.nshared), s2))))
        return rc;
  }
  // 3. dz = w (dy W2_e) act'(z1) (routed rows, dy gathered through the row -> token index,
  //    w the slot's gate weight) and (dy W2_{E+q}) act'(z1sh) (shared, output columns q H1):
  //    the GEMM applies the gate weight and the activation gradient in its epilogue and
  //    writes dz (for SwiGLU dg and du), so dh is never stored.  The same epilogue forms the
  //    combine weights' gradient dw_nj = <dy_n W2_e, h_row> as per-n-tile partials, so the
  //    expert outputs o need not be recomputed.  W2_e [M, H] is read in place as a K-major
  //    operand (k = m); z is z1, or h for ReLU (same layout: H1 = H).
  float* dwp = reinterpret_cast<float*>(ws + B.dwp);
  {
    auto p0 = routed_problem(dy, M, W2, H, M * H, ws + B.dz1, H1, static_cast<int>(H),
                             static_cast<int>(M), static_cast<int>(N), L, tiles, ntiles);
    p0.a_gather = reinterpret_cast<const int32_t*>(ws + L.tokrow);
    p0.row_scale = wrow;
    p0.hdot = ws + L.h; p0.ldh = H;
    p0.dwp = dwp; p0.dwp_ld = static_cast<int>(B.ntn);
    auto p1 = batched_problem(dy, M, W2, H, ws + B.dz1sh, Es * H1, static_cast<int>(H),
                              static_cast<int>(N), static_cast<int>(Es), BM, sa.dhsh, false);
    p0.b_kmajor = p1.b_kmajor = 1;
    p0.dact = p1.dact = 1 + c->act;
    p0.glu_h = p1.glu_h = static_cast<int>(H);
    p0.z = relu ? ws + L.h : ws + B.z1;
    p1.z = relu ? ws + L.hsh : ws + B.z1sh;
    rc = gemm(p0, Es ? &p1 : nullptr);
    if (rc) return rc;
  }
  // 6b. (second side stream, forked as soon as dz exists) dW1_e [H1, M] = dz1_e^T buf_e;
  //     shared q: dz1sh_q^T x over token ranges into partials
  {
    if ((rc = side.fork(1))) return rc;
    auto w0 = batched_problem(ws + B.dz1, H1, ws + L.buf, M, dW1, M, static_cast<int>(M),
                              static_cast<int>(H1), static_cast<int>(E), BM, sa.dw1, true);
    auto w1 = batched_problem(ws + B.dz1sh, Es * H1, x, M, shp1, M, static_cast<int>(M),
                              static_cast<int>(H1), nsh, BM, sa.dw1 + E, true);
    w0.a_kmajor = w0.b_kmajor = w1.a_kmajor = w1.b_kmajor = 1;
    if ((rc = gemm(w0, Es ? &w1 : nullptr, s3))) return rc;
    for (int64_t q = 0; q < Es; ++q)
      if ((rc = status_of(moe::launch_split_reduce(shp1 + q * B.nshared * H1 * M,
                                                   dW1 + (E + q) * H1 * M, H1 * M,
                                                   static_cast<int>(B.nshared), s3))))
        return rc;
  }
  {
    // dw_nj = sum of the row's n-tile partials (0 for dropped slots)
    rc = status_of(moe::launch_dw_reduce(m->row, dwp, reinterpret_cast<float*>(ws + B.dw),
                                         N * k, static_cast<int>(B.ntn), s));
    if (rc) return rc;
  }
  // 5a. router backward: dl from the combine weights' gradient, then dlp = dl in the layer
  //     dtype (zero-padded to Ep), the A operand of both router GEMMs below
  moe::RouterBwdArgs ra{};
  ra.logits = m->logits; ra.topk_idx = m->topk_idx;
  ra.dw = reinterpret_cast<const float*>(ws + B.dw);
  ra.Cg = reinterpret_cast<const int32_t*>(ws + L.Cg);
  ra.dl = reinterpret_cast<float*>(ws + B.dl);
  ra.coef_aux = coef_aux; ra.coef_z = coef_z; ra.coef_dev = coef_dev; ra.norm_p = c->norm_p;
  ra.N = static_cast<int>(N); ra.E = static_cast<int>(E); ra.k = static_cast<int>(k);
  ra.G = c->n_groups; ra.S = static_cast<int>(L.S); ra.norm = c->gate_norm;
  ra.n_eg = c->expert_groups;
  rc = status_of(moe::launch_router_bwd(ra, s));
  if (rc) return rc;
  {
    moe::RouterPrepArgs pa{ra.dl, ws + B.dlp, static_cast<int>(N), static_cast<int>(E),
                           static_cast<int>(B.Ep), dt};
    rc = status_of(moe::launch_router_dgrad_prep(pa, s));
    if (rc) return rc;
  }
  // 4. dx rows = dz W1_e (routed); shared: dz_sh W1_sh over k = (q, h'), whose K-major rows
  //    are the consecutive rows of W1_{E..E+Es-1}.  The router term dxrt = dl Wg reads Wg
  //    [E, M] in place as a K-major operand (k = e, K = E; dlp's zero padding and the operand
  //    bounds cover the chunk past E); without shared experts it is this launch's second
  //    problem, otherwise a launch of its own.
  {
    auto p0 = routed_problem(ws + B.dz1, H1, W1, M, H1 * M, ws + B.dbuf, M,
                             static_cast<int>(M), static_cast<int>(H1), a_rows, L, tiles, ntiles);
    p0.b_kmajor = 1;
    auto psh = dense_problem(ws + B.dz1sh, Es * H1, W1c + E * H1 * M * esz, M, ws + L.osh, M,
                             static_cast<int>(M), static_cast<int>(Es * H1),
                             static_cast<int>(N), BM);
    psh.b_kmajor = 1;
    auto prt = dense_problem(ws + B.dlp, B.Ep, Wg, M, ws + B.dxrt, M, static_cast<int>(M),
                             static_cast<int>(E), static_cast<int>(N), BM);
    prt.b_kmajor = 1;
    rc = gemm(p0, Es ? &psh : &prt);
    if (rc) return rc;
    if (Es && (rc = gemm(prt, nullptr))) return rc;
  }
  // 5b. dx = [res] dy + the kept rows' dx + shared + router term; dbg
  {
    moe::DxArgs da{dy, ws + B.dbuf, Es ? ws + L.osh : nullptr, ws + B.dxrt, m->row, dx,
                   static_cast<int>(N), static_cast<int>(M), static_cast<int>(k), c->residual,
                   dt};
    rc = status_of(moe::launch_dx_final(da, s));
    if (rc) return rc;
    moe::DwgArgs wa{ra.dl, reinterpret_cast<float*>(ws + B.partb), dbg, static_cast<int>(N),
                    static_cast<int>(E), static_cast<int>(B.nchunks)};
    rc = status_of(moe::launch_dbg(wa, s));
    if (rc) return rc;
  }
  // 6c. dWg, then the join with the side streams
  {
    // dWg [E, M] = dl^T x: token ranges into fp32 partials, then their sum in range order
    float* part = reinterpret_cast<float*>(ws + B.dwgp);
    auto p = batched_problem(ws + B.dlp, B.Ep, x, M, part, M, static_cast<int>(M),
                             static_cast<int>(E), static_cast<int>(B.nsplit), BM, sa.dwg, true);
    p.a_kmajor = 1; p.b_kmajor = 1;
    if ((rc = gemm(p, nullptr))) return rc;
    if ((rc = status_of(moe::launch_split_reduce(part, dWg, E * M, static_cast<int>(B.nsplit), s))))
      return rc;
  }
  return side.join();
}

}  // namespace

namespace moe {
int forward_workspace(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                      const void* W1, const void* W2, const float* u, void* y, float* aux,
                      const moe_meta* m, void* workspace, size_t wbytes, void* stream,
                      bool check_only) {
  return forward_impl(cfg, x, Wg, bg, W1, W2, u, y, aux, m, workspace, wbytes, stream, nullptr,
                      check_only);
}
}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid argument (cfg, NULL or misaligned pointer)";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EUNSUPPORTED: return "shape outside the kernels' constraints";
    case MOE_EHIP: return "HIP launch error";
    case MOE_ESCRATCH:
      return "layer needs more workspace than moe_forward_noalloc's static scratch "
             "(MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error";
  }
}

int moe_workspace_size(const moe_cfg* cfg, size_t* bytes) {
  if (!bytes) return MOE_EINVAL;
  Layout L;
  const int rc = make_layout(cfg, &L);
  if (rc) return rc;
  *bytes = L.total;
  return MOE_OK;
}

int moe_forward(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                const void* W1, const void* W2, const float* u, void* y, float* aux_loss,
                const moe_meta* meta, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta, workspace, workspace_bytes,
                      stream, nullptr);
}

int moe_forward_timed(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                      const void* W1, const void* W2, const float* u, void* y,
                      float* aux_loss, const moe_meta* meta, void* workspace,
                      size_t workspace_bytes, void* stream, void* const* events) {
  if (!events) return MOE_EINVAL;
  return forward_impl(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta, workspace, workspace_bytes,
                      stream, events);
}

int moe_backward_workspace_size(const moe_cfg* cfg, size_t* bytes) {
  if (!bytes) return MOE_EINVAL;
  BwdLayout B;
  const int rc = make_bwd_layout(cfg, &B);
  if (rc) return rc;
  *bytes = B.total;
  return MOE_OK;
}

int moe_forward_train(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                      const void* W1, const void* W2, const float* u, void* y, float* aux_loss,
                      const moe_meta* meta, void* workspace, size_t workspace_bytes,
                      void* stream) {
  BwdLayout B;
  const int rc = make_bwd_layout(cfg, &B);
  if (rc) return rc;
  if (!workspace || !aligned16(workspace)) return MOE_EINVAL;
  if (workspace_bytes < B.total) return MOE_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const TrainOut t{ws + B.z1, ws + B.z1sh};
  return forward_impl(cfg, x, Wg, bg, W1, W2, u, y, aux_loss, meta, workspace, workspace_bytes,
                      stream, nullptr, false, &t);
}

int moe_backward_saved(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                       const void* W1, const void* W2, const float* u, const void* dy,
                       float coef_aux, float coef_z, float coef_dev, void* dx, float* dWg,
                       float* dbg, float* dW1, float* dW2, const moe_meta* meta,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z, coef_dev, dx, dWg, dbg,
                       dW1, dW2, meta, workspace, workspace_bytes, stream, true);
}

int moe_backward(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                 const void* W1, const void* W2, const float* u, const void* dy, float coef_aux,
                 float coef_z, float coef_dev, void* dx, float* dWg, float* dbg, float* dW1,
                 float* dW2, const moe_meta* meta, void* workspace, size_t workspace_bytes,
                 void* stream) {
  return backward_impl(cfg, x, Wg, bg, W1, W2, u, dy, coef_aux, coef_z, coef_dev, dx, dWg, dbg,
                       dW1, dW2, meta, workspace, workspace_bytes, stream);
}

int moe_route(const moe_cfg* cfg, const float* logits, const float* u, const moe_meta* meta,
              float* aux_loss, void* workspace, size_t workspace_bytes, void* stream) {
  Run r;
  r.c = cfg;
  int rc = make_layout(cfg, &r.L);
  if (rc) return rc;
  if (!aux_loss || !aligned16(aux_loss) || !workspace || !aligned16(workspace))
    return MOE_EINVAL;
  if (workspace_bytes < r.L.total) return MOE_EWORKSPACE;
  if (cfg->n_tokens == 0) {
    rc = check_meta_empty(meta);
    if (rc) return rc;
    return empty_call(cfg, meta, aux_loss, static_cast<hipStream_t>(stream), nullptr);
  }
  rc = check_meta(meta, false);
  if (rc) return rc;
  if (cfg->random_routing && (!u || !aligned16(u))) return MOE_EINVAL;
  if (!logits || !aligned16(logits)) return MOE_EINVAL;
  r.ws = static_cast<char*>(workspace);
  r.s = static_cast<hipStream_t>(stream);
  rc = run_routing(r, nullptr, nullptr, nullptr, u, logits, meta, r.L.BM, nullptr, false);
  if (rc) return rc;
  moe::CombineArgs ca = combine_args(r, nullptr, nullptr, aux_loss, meta);
  return status_of(moe::launch_aux_only(ca, r.s));
}

}  // extern "C"
