// moe_router: router logits, softmax, top-k, gate weights, random routing, block histograms.
//
// [MegaBlocks] "2. 路由器：一个线性层的全部戏份": the router is a bias-free linear layer
// [tokens, M] -> [tokens, E] followed by softmax and top-k, returning the full-E scores for
// the balance loss, the top-k weights and the top-k expert ids.  [Lec16] "MoE Kernel 优化":
// the gating work (softmax, top-k, dispatch bookkeeping) runs fused in one kernel.
//
// One block = 256 threads (4 waves) = 64 consecutive tokens of one group.
//  1. GEMM: x[64, M] . Wg[E, M]^T, K staged through LDS in 256-byte row chunks (XOR-swizzled
//     16-byte columns).  bf16: v_mfma_f32_32x32x16_bf16 tiles, fp32 accumulation.  fp32:
//     plain FMA (fp32 MFMA and fp32 vector peaks are equal on this chip).
//  2. Epilogue, 4 lanes per token: + bg, logits out, row max and sum of exp (fp32), top-k
//     on the logits (ties to the lower expert index), gate weights, the random-routing
//     decision in fp64, LDS histograms of selections and active slots per rank, and the
//     per-expert column sums of the softmax probabilities (fp64) for the aux loss.
#include <math.h>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 256;  // bytes of K per LDS row per chunk

__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

__host__ __device__ inline int router_stage_bytes(int epad) {
  return kRouteTokens * kRowBytes + epad * kRowBytes;  // >= lg tile [64][epad+1] floats
}

// x[64 tokens, M] . Wg[E, M]^T -> lg[64][ls] (bf16 inputs, MFMA 32x32x16).
__device__ void router_gemm_bf16(const RouterArgs& a, unsigned char* stage, float* lg, int ls,
                                 int tok0, int nt, int epad) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int E = a.E;
  const size_t rowbytes = static_cast<size_t>(a.M) * 2;
  const int nks = static_cast<int>(rowbytes / kRowBytes);
  const char* xb = static_cast<const char*>(a.x);
  const char* wb = static_cast<const char*>(a.Wg);
  unsigned char* xs = stage;
  unsigned char* ws = stage + kRouteTokens * kRowBytes;
  const int ntiles = 2 * (epad / 32);     // 2 token tiles x (epad/32) expert tiles
  const int wl = epad / 16;               // Wg 16-byte chunks per thread per K chunk

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  u32x4 xr[4];
  u32x4 wr[16];

  auto load = [&](int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = t + kThreads * i, r = idx >> 4, c = idx & 15;
      const int rr = r < nt ? r : nt - 1;
      xr[i] = *reinterpret_cast<const u32x4*>(xb + static_cast<size_t>(tok0 + rr) * rowbytes +
                                              static_cast<size_t>(kc) * kRowBytes + c * 16);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < wl) {
        const int idx = t + kThreads * i, r = idx >> 4, c = idx & 15;
        const int re = r < E ? r : E - 1;
        wr[i] = *reinterpret_cast<const u32x4*>(wb + static_cast<size_t>(re) * rowbytes +
                                                static_cast<size_t>(kc) * kRowBytes + c * 16);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = t + kThreads * i, r = idx >> 4, c = idx & 15;
      *reinterpret_cast<u32x4*>(xs + r * kRowBytes + swz(r, c) * 16) = xr[i];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < wl) {
        const int idx = t + kThreads * i, r = idx >> 4, c = idx & 15;
        *reinterpret_cast<u32x4*>(ws + r * kRowBytes + swz(r, c) * 16) = wr[i];
      }
    }
  };

  load(0);
  for (int kc = 0; kc < nks; ++kc) {
    store();
    __syncthreads();
    if (kc + 1 < nks) load(kc + 1);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tile = w + 4 * i;
        if (tile < ntiles) {
          const int ra = (tile & 1) * 32 + (lane & 31);
          const int rb = (tile >> 1) * 32 + (lane & 31);
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(xs + ra * kRowBytes + swz(ra, c) * 16);
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(ws + rb * kRowBytes + swz(rb, c) * 16);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  // The loop ended with a barrier, so lg (aliasing the staging area) can be written.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tile = w + 4 * i;
    if (tile < ntiles) {
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
  const int t = threadIdx.x, tl = t & 63, eg = t >> 6;
  const int E = a.E;
  const size_t rowbytes = static_cast<size_t>(a.M) * 4;
  const int nks = static_cast<int>(rowbytes / kRowBytes);
  const char* xb = static_cast<const char*>(a.x);
  const char* wb = static_cast<const char*>(a.Wg);
  unsigned char* xs = stage;
  unsigned char* ws = stage + kRouteTokens * kRowBytes;
  const int wl = epad / 16;
  const int ne = epad / 4;               // experts per thread: e = eg + 4 i

  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;

  for (int kc = 0; kc < nks; ++kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = t + kThreads * i, r = idx >> 4, c = idx & 15;
      const int rr = r < nt ? r : nt - 1;
      *reinterpret_cast<u32x4*>(xs + r * kRowBytes + swz(r, c) * 16) =
          *reinterpret_cast<const u32x4*>(xb + static_cast<size_t>(tok0 + rr) * rowbytes +
                                          static_cast<size_t>(kc) * kRowBytes + c * 16);
    }
    for (int i = 0; i < wl; ++i) {
      const int idx = t + kThreads * i, r = idx >> 4, c = idx & 15;
      const int re = r < E ? r : E - 1;
      *reinterpret_cast<u32x4*>(ws + r * kRowBytes + swz(r, c) * 16) =
          *reinterpret_cast<const u32x4*>(wb + static_cast<size_t>(re) * rowbytes +
                                          static_cast<size_t>(kc) * kRowBytes + c * 16);
    }
    __syncthreads();
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
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 64; ++i)
    if (i < ne) lg[tl * ls + eg + 4 * i] = acc[i];
}

template <int DT>
__global__ __launch_bounds__(kThreads) void router_kernel(RouterArgs a, int epad) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int t = threadIdx.x;
  const int b = blockIdx.x;
  const int g = b / a.nbg, bi = b - g * a.nbg;
  const int tok0 = g * a.S + bi * kRouteTokens;
  const int nt = min(kRouteTokens, a.S - bi * kRouteTokens);
  const int E = a.E, k = a.k;
  const int ls = epad + 1;
  float* lg = reinterpret_cast<float*>(smem);
  int* hsel = reinterpret_cast<int*>(smem + router_stage_bytes(epad));
  int* hact = hsel + epad;
  for (int i = t; i < epad * (1 + k); i += kThreads) hsel[i] = 0;

  if (a.logits_in) {
    for (int idx = t; idx < kRouteTokens * E; idx += kThreads) {
      const int r = idx / E, e = idx - r * E;
      lg[r * ls + e] = r < nt ? a.logits_in[static_cast<size_t>(tok0 + r) * E + e] : 0.f;
    }
    __syncthreads();
  } else {
    if (DT == 1)
      router_gemm_bf16(a, smem, lg, ls, tok0, nt, epad);
    else
      router_gemm_f32(a, smem, lg, ls, tok0, nt, epad);
    __syncthreads();
    for (int idx = t; idx < nt * E; idx += kThreads) {
      const int r = idx / E, e = idx - r * E;
      float v = lg[r * ls + e];
      if (a.bg) v += a.bg[e];
      lg[r * ls + e] = v;
      if (a.logits_out) a.logits_out[static_cast<size_t>(tok0 + r) * E + e] = v;
    }
    __syncthreads();
  }

  // ---- per token: 4 lanes (a quad) share one row of logits
  const int tl = t >> 2, q = t & 3;
  const bool valid = tl < nt;
  const int n = tok0 + tl;
  float* row = lg + tl * ls;

  float mx = -INFINITY;
  for (int e = q; e < E; e += 4) mx = fmaxf(mx, row[e]);
  mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
  float se = 0.f;
  for (int e = q; e < E; e += 4) se += expf(row[e] - mx);
  se += __shfl_xor(se, 1, 64);
  se += __shfl_xor(se, 2, 64);

  int sel_e[kMaxTopK];
  float sel_l[kMaxTopK];
  uint64_t taken = 0;  // bit i <-> expert q + 4 i already selected
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    sel_e[j] = 0;
    sel_l[j] = 0.f;
    if (j < k) {
      float bv = -INFINITY;
      int bix = 0x7fffffff;
      int i = 0;
      for (int e = q; e < E; e += 4, ++i) {
        if (!((taken >> i) & 1ull)) {
          float v = row[e];
          if (v != v) v = -INFINITY;  // a NaN never wins, so bix is always a real expert
          if (v > bv || (v == bv && e < bix)) { bv = v; bix = e; }
        }
      }
#pragma unroll
      for (int off = 1; off <= 2; off <<= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bix, off, 64);
        if (ov > bv || (ov == bv && oi < bix)) { bv = ov; bix = oi; }
      }
      sel_e[j] = bix;
      sel_l[j] = bv;
      if ((bix & 3) == q) taken |= 1ull << (bix >> 2);
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
  if (a.norm) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) wgt[j] = wgt[j] / psel;
  }
  // [GShard] "Random routing": keep the 2nd slot iff u < 2 w2, w2 = 1 / (1 + exp(l1 - l2)),
  // decided in fp64 from the two fp32 logits.
  bool keep2 = true;
  if (a.rr && valid) {
    const double th = 2.0 / (1.0 + exp(static_cast<double>(sel_l[0]) - static_cast<double>(sel_l[1])));
    keep2 = static_cast<double>(a.u[n]) < th;
  }

  if (valid) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k && (j & 3) == q) {
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
  for (int e = q; e < E; e += 4) row[e] = valid ? expf(row[e] - mx) / se : 0.f;
  __syncthreads();

  for (int e = t; e < E; e += kThreads) {
    double s = 0.0;
    for (int r = 0; r < nt; ++r) s += static_cast<double>(lg[r * ls + e]);
    const size_t o = (static_cast<size_t>(g) * E + e) * a.nbg + bi;
    a.psum[o] = s;
    a.sel[o] = hsel[e];
  }
  for (int idx = t; idx < k * E; idx += kThreads) {
    const int j = idx / E, e = idx - j * E;
    a.ahist[((static_cast<size_t>(g) * k + j) * E + e) * a.nbg + bi] = hact[j * epad + e];
  }
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t s) {
  const int epad = (a.E + 31) / 32 * 32;
  const size_t lds = router_stage_bytes(epad) + static_cast<size_t>(epad) * (1 + a.k) * 4;
  const int grid = a.G * a.nbg;
  if (grid == 0) return hipSuccess;
  if (a.dtype == 1) {
    static bool attr = false;
    if (!attr) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(&router_kernel<1>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr = true;
    }
    hipLaunchKernelGGL(router_kernel<1>, dim3(grid), dim3(kThreads), lds, s, a, epad);
  } else {
    static bool attr = false;
    if (!attr) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(&router_kernel<0>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      attr = true;
    }
    hipLaunchKernelGGL(router_kernel<0>, dim3(grid), dim3(kThreads), lds, s, a, epad);
  }
  return hipGetLastError();
}

}  // namespace moe
