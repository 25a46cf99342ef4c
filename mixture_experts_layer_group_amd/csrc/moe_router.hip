// moe_router: router logits, softmax, top-k, gate weights, random routing, block histograms.
//
// [MegaBlocks] "2. 路由器：一个线性层的全部戏份": the router is a bias-free linear layer
// [tokens, M] -> [tokens, E] followed by softmax and top-k, returning the full-E scores for
// the balance loss, the top-k weights and the top-k expert ids.  [Lec16] "MoE Kernel 优化":
// the gating work (softmax, top-k, dispatch bookkeeping) runs fused in one kernel.
//
// One block = 64 consecutive tokens of one group, on 1024 threads (16 waves, one block per
// CU), or, for bf16 launches with more blocks than CUs and E <= 128, on 512 threads (8
// waves) within 80 KB of LDS, so that two blocks share a CU and one's epilogue runs beside
// the other's GEMM phase.
//  1. GEMM on waves 0..3: x[64, M] . Wg[E, M]^T.  bf16: both operands stream global -> LDS
//     directly (buffer_load ... lds) through 2-4 stages of 256- or 128-byte row chunks
//     (XOR-swizzled 16-byte columns) into v_mfma_f32_32x32x16_bf16 tiles, fp32
//     accumulation.  fp32: plain FMA through an LDS staging area (fp32 MFMA and fp32
//     vector peaks are equal on this chip).
//  2. Epilogue, 16 (or 8) lanes per token (all waves): + bg, logits out, row max and sum of exp
//     (fp32), top-k on the logits (ties to the lower expert index), gate weights (sum or
//     p-norm), the random-routing decision in fp64, LDS histograms of selections and
//     active slots per rank, the per-expert column sums of the softmax probabilities
//     (fp64) for the aux loss, and the block's sum of logsumexp^2 (fp64) for the z-loss.
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;       // 16 waves: all of them share the per-token epilogue
// Launches with more router blocks than the chip has CUs (bf16, E <= 128): 8 waves and at
// most 80 KB of LDS per block, so that two blocks share a CU and one block's epilogue runs
// beside the other's GEMM phase.
constexpr int kThreadsPair = 512;
constexpr int kChipCUs = 256;
constexpr int kGemmThreads = 256;    // the GEMM phase runs on waves 0..3
constexpr int kRowBytes = 256;  // bytes of K per LDS row per chunk

}  // namespace
__host__ __device__ int router_lds_stage_bytes(int dt, int epad, int nt);
namespace {

__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

// LDS staging area of the fp32 path: x[64] and Wg[epad] rows of 256 bytes (it is also
// large enough for the logits tile [64][epad + 1] floats that aliases it afterwards).
__host__ __device__ inline int router_stage_bytes(int epad) {
  return kRouteTokens * kRowBytes + epad * kRowBytes;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           0x00020000);
}

// 16 bytes per lane from a raw buffer straight into LDS (lane i -> lds + 16 i).
__device__ __forceinline__ void dma16(rsrc_t r, unsigned char* lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS layout of the bf16 router GEMM for EPAD padded experts and top-k <= 8: stages of
// x[64] + Wg[EPAD] rows of ROWB bytes, within LDSB bytes together with the histograms
// (256-byte rows unless fewer than two such stages fit).
template <int EPAD, int LDSB>
struct RouterPipe {
  static constexpr int kHist = EPAD * (1 + kMaxTopK) * 4;
  static constexpr int kRowB =
      EPAD >= 256 || (LDSB - kHist) / ((kRouteTokens + EPAD) * 256) < 2 ? 128 : 256;
  static constexpr int kStage = (kRouteTokens + EPAD) * kRowB;
  static constexpr int kFit = (LDSB - kHist) / kStage;
  static constexpr int kStages = kFit >= 4 ? 4 : kFit;
  static constexpr int kXq = kRouteTokens * kRowB / 1024 / 4;  // x loads per wave per chunk
  static constexpr int kWq = EPAD * kRowB / 1024 / 4;          // Wg loads per wave per chunk
  static_assert(kStages >= 2, "router pipeline needs two stages");
};

// XOR pattern of the 16-byte columns of row r: conflict-free fragment reads of one column
// from 16 consecutive rows on the 64-bank LDS (16 columns per 256-byte row, or 8 per 128-byte
// row with two rows per bank line).
template <int ROWB>
__device__ __forceinline__ int rswz(int r) {
  return ROWB == 256 ? (r & 15) : (((r >> 1) & 7) ^ ((r & 1) << 2));
}

// x[64 tokens, M] . Wg[E, M]^T -> lg[64][ls] (bf16, v_mfma_f32_32x32x16_bf16, fp32 sums).
// K is streamed in row chunks of ROWB bytes through RouterPipe::kStages LDS stages, each
// filled by buffer_load ... lds (lane i of a wave instruction -> 16 bytes at LDS unit i), so
// several chunks are in flight while one is multiplied.  The 16-byte columns of each row are
// XOR-permuted (rswz, applied on the global side) so fragment reads are conflict-free.  Rows
// of x past the block's tokens and rows of Wg past E read as zeros (buffer bounds).
template <int EPAD, int LDSB>
__device__ void router_gemm_bf16(const RouterArgs& a, unsigned char* smem, float* lg, int ls,
                                 int tok0, int nt) {
  using P = RouterPipe<EPAD, LDSB>;
  constexpr int NST = P::kStages, STAGE = P::kStage, XQ = P::kXq, WQ = P::kWq;
  constexpr int ROWB = P::kRowB, CPR = ROWB / 16;
  constexpr int NTILE = 2 * (EPAD / 32);   // 2 token tiles x EPAD/32 expert tiles
  constexpr int TPW = (NTILE + 3) / 4;     // MFMA tiles per wave
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int E = a.E;
  const uint32_t rowbytes = static_cast<uint32_t>(a.M) * 2;
  const int nks = static_cast<int>(rowbytes / ROWB);
  const char* xb = static_cast<const char*>(a.x) + static_cast<size_t>(tok0) * rowbytes;
  const rsrc_t xr = make_rsrc(xb, static_cast<int64_t>(nt) * rowbytes);
  const rsrc_t wr = make_rsrc(a.Wg, static_cast<int64_t>(E) * rowbytes);

  uint32_t xoff[XQ], woff[WQ];
#pragma unroll
  for (int q = 0; q < XQ; ++q) {
    const int u = (w + 4 * q) * 64 + lane, r = u / CPR, c = (u % CPR) ^ rswz<ROWB>(r);
    xoff[q] = r * rowbytes + c * 16;
  }
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int u = (w + 4 * q) * 64 + lane, r = u / CPR, c = (u % CPR) ^ rswz<ROWB>(r);
    woff[q] = r * rowbytes + c * 16;
  }
  auto issue = [&](int kc, int st) {
    unsigned char* xs = smem + st * STAGE;
    unsigned char* ws = xs + kRouteTokens * ROWB;
    const uint32_t k0 = static_cast<uint32_t>(kc) * ROWB;
#pragma unroll
    for (int q = 0; q < XQ; ++q) dma16(xr, xs + (w + 4 * q) * 1024, xoff[q], k0);
#pragma unroll
    for (int q = 0; q < WQ; ++q) dma16(wr, ws + (w + 4 * q) * 1024, woff[q], k0);
  };

  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = f32x16{};
  const int sw = rswz<ROWB>(lane & 31);
  auto compute = [&](int st) {
    const unsigned char* xs = smem + st * STAGE;
    const unsigned char* ws = xs + kRouteTokens * ROWB;
#pragma unroll
    for (int s = 0; s < ROWB / 32; ++s) {
      const int phys = ((2 * s + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tile = w + 4 * i;
        if (tile < NTILE) {
          const int ra = (tile & 1) * 32 + (lane & 31);
          const int rb = (tile >> 1) * 32 + (lane & 31);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(xs + ra * ROWB + phys);
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(ws + rb * ROWB + phys);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i], 0, 0, 0);
        }
      }
    }
  };

  // Waves 0..3 load and multiply; the other waves of the block only take part in the barriers
  // (they issue no loads, so their vmcnt waits return at once).
  const bool gw = w < 4;
  const int pre = nks < NST - 1 ? nks : NST - 1;
  if (gw)
    for (int i = 0; i < pre; ++i) issue(i, i);
  for (int kc = 0; kc < nks; ++kc) {
    // chunks issued after chunk kc: min(NST - 2, nks - 1 - kc)
    const int after = nks - 1 - kc < NST - 2 ? nks - 1 - kc : NST - 2;
    if (after >= 2) MOE_WAIT_VMCNT(2 * (XQ + WQ));
    else if (after == 1) MOE_WAIT_VMCNT(XQ + WQ);
    else MOE_WAIT_VMCNT(0);
    lds_barrier();
    if (gw) {
      if (kc + NST - 1 < nks) issue(kc + NST - 1, (kc + NST - 1) % NST);
      compute(kc % NST);
    }
  }
  lds_barrier();  // every wave is done with the stages before lg (aliasing them) is written
  if (!gw) return;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = w + 4 * i;
    if (tile < NTILE) {
      const int col = (tile >> 1) * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (tile & 1) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        lg[row * ls + col] = acc[i][r];
      }
    }
  }
}

// Same contraction for fp32 inputs with plain FMAs: lane = token, wave = expert phase.
__device__ void router_gemm_f32(const RouterArgs& a, unsigned char* stage, float* lg, int ls,
                                int tok0, int nt, int epad) {
  const int t = threadIdx.x, tl = t & 63, eg = (t >> 6) & 3;
  const int E = a.E;
  const size_t rowbytes = static_cast<size_t>(a.M) * 4;
  const int nks = static_cast<int>(rowbytes / kRowBytes);
  const char* xb = static_cast<const char*>(a.x);
  const char* wb = static_cast<const char*>(a.Wg);
  unsigned char* xs = stage;
  unsigned char* ws = stage + kRouteTokens * kRowBytes;
  const int wl = epad / 16;
  const int ne = epad / 4;               // experts per thread: e = eg + 4 i

  const bool gt = t < kGemmThreads;  // threads 0..255 compute; the rest join the barriers
  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;

  for (int kc = 0; kc < nks; ++kc) {
    if (gt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int idx = t + kGemmThreads * i, r = idx >> 4, c = idx & 15;
        const int rr = r < nt ? r : nt - 1;
        *reinterpret_cast<u32x4*>(xs + r * kRowBytes + swz(r, c) * 16) =
            *reinterpret_cast<const u32x4*>(xb + static_cast<size_t>(tok0 + rr) * rowbytes +
                                            static_cast<size_t>(kc) * kRowBytes + c * 16);
      }
      for (int i = 0; i < wl; ++i) {
        const int idx = t + kGemmThreads * i, r = idx >> 4, c = idx & 15;
        const int re = r < E ? r : E - 1;
        *reinterpret_cast<u32x4*>(ws + r * kRowBytes + swz(r, c) * 16) =
            *reinterpret_cast<const u32x4*>(wb + static_cast<size_t>(re) * rowbytes +
                                            static_cast<size_t>(kc) * kRowBytes + c * 16);
      }
    }
    __syncthreads();
    if (gt) {
      for (int c = 0; c < 16; ++c) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(xs + tl * kRowBytes + swz(tl, c) * 16);
#pragma unroll
        for (int i = 0; i < 64; ++i) {
          if (i < ne) {
            const int e = eg + 4 * i;
            const f32x4 wv = *reinterpret_cast<const f32x4*>(ws + e * kRowBytes + swz(e, c) * 16);
            acc[i] = fmaf(xv[0], wv[0], acc[i]);
            acc[i] = fmaf(xv[1], wv[1], acc[i]);
            acc[i] = fmaf(xv[2], wv[2], acc[i]);
            acc[i] = fmaf(xv[3], wv[3], acc[i]);
          }
        }
      }
    }
    __syncthreads();
  }
  if (!gt) return;
#pragma unroll
  for (int i = 0; i < 64; ++i)
    if (i < ne) lg[tl * ls + eg + 4 * i] = acc[i];
}

template <int DT, int EPAD, int NT>
__global__ __launch_bounds__(NT, NT == kThreads ? 1 : 2) void router_kernel(RouterArgs a) {
  constexpr int epad = EPAD;
  constexpr int LDSB = (NT == kThreads ? 160 : 80) * 1024;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int t = threadIdx.x;
  const int b = blockIdx.x;
  const int g = b / a.nbg, bi = b - g * a.nbg;
  const int tok0 = g * a.S + bi * kRouteTokens;
  const int nt = min(kRouteTokens, a.S - bi * kRouteTokens);
  const int E = a.E, k = a.k;
  const int ls = epad + 1;
  float* lg = reinterpret_cast<float*>(smem);
  int* hsel = reinterpret_cast<int*>(smem + router_lds_stage_bytes(DT, epad, NT));
  int* hact = hsel + epad;
  for (int i = t; i < epad * (1 + k); i += NT) hsel[i] = 0;

  if (a.logits_in) {
    for (int idx = t; idx < kRouteTokens * E; idx += NT) {
      const int r = idx / E, e = idx - r * E;
      lg[r * ls + e] = r < nt ? a.logits_in[static_cast<size_t>(tok0 + r) * E + e] : 0.f;
    }
    __syncthreads();
  } else {
    if (DT == 1)
      router_gemm_bf16<EPAD, LDSB>(a, smem, lg, ls, tok0, nt);
    else
      router_gemm_f32(a, smem, lg, ls, tok0, nt, epad);
    __syncthreads();
    for (int idx = t; idx < nt * E; idx += NT) {
      const int r = idx / E, e = idx - r * E;
      float v = lg[r * ls + e];
      if (a.bg) v += a.bg[e];
      lg[r * ls + e] = v;
      if (a.logits_out) a.logits_out[static_cast<size_t>(tok0 + r) * E + e] = v;
    }
    __syncthreads();
  }

  // ---- per token: L = 16 (or 8) consecutive lanes share one row of logits
  constexpr int L = NT / kRouteTokens;
  const int tl = t / L, q = t % L;
  const bool valid = tl < nt;
  const int n = tok0 + tl;
  float* row = lg + tl * ls;

  static_assert(L == 16 || L == 8, "one token per 16- or 8-lane DPP group");
  // The lane's logits (experts q + L i) stay in registers for the max, the sum and top-k.
  constexpr int NV = EPAD / L;
  float rv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) rv[i] = q + L * i < E ? row[q + L * i] : -INFINITY;
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (q + L * i < E) mx = fmaxf(mx, rv[i]);
  mx = group_max<L>(mx);
  float se = 0.f;
  float ev[NV];   // exp(l - max), kept for the probabilities below
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    ev[i] = q + L * i < E ? expf(rv[i] - mx) : 0.f;
    se += ev[i];
  }
  se = group_sum<L>(se);

  // Group-limited routing ([Lec16] "DeepSeek V3 MoE (670B)"): the E experts form n_eg
  // contiguous groups; a group scores its best logit, and the topk_eg best groups (ties to
  // the lower index) stay open.  Lane q scores groups q + L h (up to 32 groups).
  uint32_t taken = 0;  // bit i <-> expert q + L i excluded (E <= 256 -> i < 32)
  if (a.n_eg > 1) {
    const int D = a.n_eg, gs = E / D;
    constexpr int NG = 32 / L;
    float gv[NG];
#pragma unroll
    for (int h = 0; h < NG; ++h) {
      const int d = q + h * L;
      float v = -INFINITY;
      if (d < D)
        for (int i = 0; i < gs; ++i) {
          const float x = row[d * gs + i];
          v = x != x ? v : fmaxf(v, x);  // NaN never scores
        }
      gv[h] = v;
    }
    uint32_t open = 0;
    for (int r = 0; r < a.topk_eg; ++r) {
      float bv = -INFINITY;
      int bd = 0x7fffffff;
#pragma unroll
      for (int h = 0; h < NG; ++h) {
        const int d = q + h * L;
        if (d < D && !((open >> d) & 1u) && (gv[h] > bv || (gv[h] == bv && d < bd))) {
          bv = gv[h];
          bd = d;
        }
      }
      group_argmax<L>(bv, bd);
      open |= 1u << bd;
    }
    // experts of closed groups are excluded, so the top-k below never picks them
    int i = 0;
    for (int e = q; e < E; e += L, ++i)
      if (!((open >> (e / gs)) & 1u)) taken |= 1u << i;
  }

  // k rounds of argmax over the candidates (bit i <-> expert q + L i, not yet taken and below
  // E).  The comparisons are selects, not branches: a divergent branch per element would cost
  // an exec-mask save, test and restore each.  A NaN logit scores -inf, so it never beats a
  // number, and ties (also among -inf) go to the lower expert index, so bix is always a real
  // candidate.
  float rk[NV];
  uint32_t cand = ~taken;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    rk[i] = rv[i] != rv[i] ? -INFINITY : rv[i];
    if (q + L * i >= E) cand &= ~(1u << i);
  }
  int sel_e[kMaxTopK];
  float sel_l[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    sel_e[j] = 0;
    sel_l[j] = 0.f;
    if (j < k) {
      float bv = -INFINITY;
      int bix = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = q + L * i;
        const bool better = ((cand >> i) & 1u) & ((rk[i] > bv) | ((rk[i] == bv) & (e < bix)));
        bv = better ? rk[i] : bv;
        bix = better ? e : bix;
      }
      group_argmax<L>(bv, bix);
      sel_e[j] = bix;
      sel_l[j] = bv;
      cand &= bix % L == q ? ~(1u << (bix / L)) : ~0u;
    }
  }

  float wgt[kMaxTopK];
  float psel = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    wgt[j] = 0.f;
    if (j < k) {
      wgt[j] = expf(sel_l[j] - mx) / se;
      psel += wgt[j];
    }
  }
  if (a.norm == 1) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) wgt[j] = wgt[j] / psel;
  } else if (a.norm == 2) {
    // [MegaBlocks] section 2: the selected weights divided by their p-norm
    float sp = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) sp += powf(wgt[j], a.norm_p);
    const float den = powf(sp, 1.0f / a.norm_p);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) wgt[j] = wgt[j] / den;
  }
  // Router z-loss term ([MegaBlocks] section 2): logsumexp of the token's logits, kept in
  // the spare last column of its LDS row until the block sums the squares.
  if (q == 0) row[epad] = valid ? mx + logf(se) : 0.f;
  // [GShard] "Random routing": keep the 2nd slot iff u < 2 w2, w2 = 1 / (1 + exp(l1 - l2)),
  // decided in fp64 from the two fp32 logits (by the two lanes that use it).
  bool keep2 = true;
  if (a.rr && valid && q < 2) {
    const double th = 2.0 / (1.0 + exp(static_cast<double>(sel_l[0]) - static_cast<double>(sel_l[1])));
    keep2 = static_cast<double>(a.u[n]) < th;
  }

  if (valid) {
    // lane q < k writes slot q
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && j == q) {
        const size_t o = static_cast<size_t>(n) * k + j;
        a.topk_idx[o] = sel_e[j];
        a.topk_w[o] = wgt[j];
        a.active[o] = (j == 1 && a.rr) ? static_cast<uint8_t>(keep2) : static_cast<uint8_t>(1);
      }
    }
    if (q == 0) {
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k) {
          atomicAdd(&hsel[sel_e[j]], 1);
          if (!(j == 1 && a.rr) || keep2) atomicAdd(&hact[j * epad + sel_e[j]], 1);
        }
      }
    }
  }
  // Softmax probabilities for the block's column sums; each lane rewrites only its own
  // entries of its own row, which no other lane reads before the barrier.
  const float inv_se = 1.0f / se;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (q + L * i < E) row[q + L * i] = valid ? ev[i] * inv_se : 0.f;
  __syncthreads();

  // Column sums of the probabilities: SPC consecutive lanes per expert, each summing every
  // SPC-th row in fp64, then a fixed butterfly over those lanes (deterministic).
  constexpr int SPC = NT / EPAD;
  {
    const int e = t / SPC, part = t % SPC;
    double s = 0.0;
    if (e < E)
      for (int r = part; r < nt; r += SPC) s += static_cast<double>(lg[r * ls + e]);
    if (SPC <= 16) {
      s = group_sum<(SPC <= 16 ? SPC : 16)>(s);
    } else {
#pragma unroll
      for (int off = 1; off < SPC; off <<= 1) s += __shfl_xor(s, off, 64);
    }
    if (e < E && part == 0) {
      const size_t o = (static_cast<size_t>(g) * E + e) * a.nbg + bi;
      a.psum[o] = s;
      a.sel[o] = hsel[e];
    }
  }
  for (int idx = t; idx < k * E; idx += NT) {
    const int j = idx / E, e = idx - j * E;
    a.ahist[((static_cast<size_t>(g) * k + j) * E + e) * a.nbg + bi] = hact[j * epad + e];
  }
  if (t < kRouteTokens) {  // one wave: the block's sum of logsumexp^2, fp64, fixed order
    double z = 0.0;
    if (t < nt) {
      const double v = lg[t * ls + epad];
      z = v * v;
    }
    z = wave_sum(z);
    if (t == 0) a.zpart[b] = z;
  }
}

template <int DT, int EPAD, int NT>
hipError_t launch_router_t(const RouterArgs& a, hipStream_t s, int grid) {
  const size_t lds =
      router_lds_stage_bytes(DT, EPAD, NT) + static_cast<size_t>(EPAD) * (1 + a.k) * 4;
  static const bool attr = [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&router_kernel<DT, EPAD, NT>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return true;
  }();
  (void)attr;
  hipLaunchKernelGGL((router_kernel<DT, EPAD, NT>), dim3(grid), dim3(NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace

// LDS bytes before the histograms: the bf16 pipeline stages (or the fp32 staging area),
// never less than the logits tile [64][epad + 1] floats that aliases them.
__host__ __device__ int router_lds_stage_bytes(int dt, int epad, int nt) {
  int b = router_stage_bytes(epad);
  if (dt == 1) {   // the layout of RouterPipe<epad, budget>
    const int budget = (nt == kThreads ? 160 : 80) * 1024;
    const int hist = epad * (1 + kMaxTopK) * 4;
    const int rowb = epad >= 256 || (budget - hist) / ((kRouteTokens + epad) * 256) < 2 ? 128 : 256;
    const int stage = (kRouteTokens + epad) * rowb;
    const int fit = (budget - hist) / stage;
    b = (fit >= 4 ? 4 : fit) * stage;
  }
  const int lgb = kRouteTokens * (epad + 1) * 4;
  return b > lgb ? b : lgb;
}

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  const int epad = (a.E + 31) / 32 * 32;
  const int grid = a.G * a.nbg;
  if (grid == 0) return hipSuccess;
  const int e = epad <= 32 ? 32 : epad <= 64 ? 64 : epad <= 128 ? 128 : 256;
  if (a.dtype == 1) {
    // more router blocks than CUs: two blocks of 8 waves per CU
    if (grid > kChipCUs && e <= 128) {
      if (e == 32) return launch_router_t<1, 32, kThreadsPair>(a, s, grid);
      if (e == 64) return launch_router_t<1, 64, kThreadsPair>(a, s, grid);
      return launch_router_t<1, 128, kThreadsPair>(a, s, grid);
    }
    if (e == 32) return launch_router_t<1, 32, kThreads>(a, s, grid);
    if (e == 64) return launch_router_t<1, 64, kThreads>(a, s, grid);
    if (e == 128) return launch_router_t<1, 128, kThreads>(a, s, grid);
    return launch_router_t<1, 256, kThreads>(a, s, grid);
  }
  if (e == 32) return launch_router_t<0, 32, kThreads>(a, s, grid);
  if (e == 64) return launch_router_t<0, 64, kThreads>(a, s, grid);
  if (e == 128) return launch_router_t<0, 128, kThreads>(a, s, grid);
  return launch_router_t<0, 256, kThreads>(a, s, grid);
}

}  // namespace moe
