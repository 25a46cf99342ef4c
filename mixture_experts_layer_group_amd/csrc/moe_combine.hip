// moe_combine: expert outputs back to token order, and the final aux-loss reduction.
//
// y_n = sum_j w_{n,j} o[row_{n,j}] + o_sh[n] + x_n (residual), in fp32 with one rounding to
// the layer dtype, summed in that order.  [GShard] "MoE Transformer": the layer output is
// the gate-weighted sum of the selected experts' outputs; "Capacity overflow 会跳过 expert
// computation": a token with no kept slot leaves through the residual, so y_n = x_n
// bit-exactly (0 + x in fp32 is x).  [Lec16] "共享专家 vs. 路由专家": the shared experts add
// with weight 1.  Lanes move 16-byte chunks of rows; a block takes as many tokens as make
// one round of two (short rows) or four chunks per lane, so that each lane issues all its
// loads at once.
//
// Block 0 also finishes the aux loss of [GShard] "Top-2 gating 的四个机制 / Auxiliary loss":
// aux = (1/G) sum_g E/(k S) sum_e m_{g,e} c_{g,e},  m_{g,e} = P_{g,e} / S, from the per-
// (group, expert) sums of probabilities P and selections c, and the router z-loss of
// [MegaBlocks] section 2, (1/N) sum_n logsumexp(logits_n)^2, from the router blocks' partial
// sums, and the device-level balance loss of [Lec16] "DeepSeek MoE 的负载均衡" (the
// expert-level terms grouped by the D expert groups: mean f times summed P per group); all
// in fp64 with fixed-order reductions (deterministic).
#include <algorithm>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kTokMax = 64;  // tokens per block at most (short rows)

// Every o row, x row and shared-expert row is read exactly once and y is written once, so
// they bypass the caches' retention (non-temporal).
template <class V>
__device__ __forceinline__ V ld_stream(const V* p) {
  return __builtin_nontemporal_load(p);
}
template <class V>
__device__ __forceinline__ void st_stream(V* p, V v) {
  __builtin_nontemporal_store(v, p);
}

__device__ void aux_final(const CombineArgs& a) {
  __shared__ double red[12];
  const int t = threadIdx.x;
  double s = 0.0, z = 0.0, dv = 0.0;
  const int n = a.G * a.E;
  for (int i = t; i < n; i += 256) s += a.Pg[i] * static_cast<double>(a.Cg[i]);
  for (int i = t; i < a.nblocks; i += 256) z += a.zpart[i];
  // device-level loss: per (token group, expert group) the selections and probability sums
  // of the group's experts, one wave per pair, its lanes over the experts
  const int gs = a.E / a.n_eg, lane = t & 63;
  for (int pr = t >> 6; pr < a.G * a.n_eg; pr += 4) {
    const int64_t base = static_cast<int64_t>(pr) * gs;  // (g, d) -> experts [d gs, +gs) of g
    double P = 0.0;
    int C = 0;
    for (int x = lane; x < gs; x += 64) {
      P += a.Pg[base + x];
      C += a.Cg[base + x];
    }
    P = wave_sum(P);
    C = wave_sum(C);
    if (lane == 0) dv += static_cast<double>(C) * P;
  }
  s = wave_sum(s);
  z = wave_sum(z);
  dv = wave_sum(dv);
  if ((t & 63) == 0) {
    red[t >> 6] = s;
    red[4 + (t >> 6)] = z;
    red[8 + (t >> 6)] = dv;
  }
  __syncthreads();
  if (t == 0) {
    const double tot = ((red[0] + red[1]) + red[2]) + red[3];
    const double S = static_cast<double>(a.S);
    const double aux = static_cast<double>(a.E) * tot / (static_cast<double>(a.G) * a.k * S * S);
    *a.aux = static_cast<float>(aux);
    if (a.z_loss) {
      const double zt = ((red[4] + red[5]) + red[6]) + red[7];
      *a.z_loss = static_cast<float>(zt / static_cast<double>(a.N));
    }
    if (a.dev_loss) {  // (1/G) sum_g sum_j (D / (k S)) C_gj (P_gj / S)
      const double dt = ((red[8] + red[9]) + red[10]) + red[11];
      *a.dev_loss = static_cast<float>(static_cast<double>(a.n_eg) * dt /
                                       (static_cast<double>(a.G) * a.k * S * S));
    }
  }
}

// KT = top-k (compile time, so that the slot loops are straight-line code); U = chunks per
// lane and round.
template <int DT, int KT, int U>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  __shared__ int rows_s[kTokMax][kMaxTopK];
  __shared__ float w_s[kTokMax][kMaxTopK];
  const int t = threadIdx.x;
  const int tok0 = blockIdx.x * a.tpb;
  const int nt = min(a.tpb, a.N - tok0);
  constexpr int k = KT;
  if (blockIdx.x == 0) aux_final(a);
  for (int i = t; i < nt * k; i += 256) {
    const int tl = i / k, jj = i - tl * k;
    const size_t o = static_cast<size_t>(tok0) * k + i;
    rows_s[tl][jj] = a.row[o];
    w_s[tl][jj] = a.topk_w[o];
  }
  __syncthreads();

  constexpr int EPC = DT == 1 ? 8 : 4;  // elements per 16-byte chunk
  const int ch = a.M / EPC;
  const size_t rowbytes = static_cast<size_t>(a.M) * (DT == 1 ? 2 : 4);
  const char* __restrict__ xb = static_cast<const char*>(a.x);
  const char* __restrict__ ob = static_cast<const char*>(a.o);
  const char* __restrict__ sb = static_cast<const char*>(a.o_sh);
  char* __restrict__ yb = static_cast<char*>(a.y);
  auto add = [&](float (&acc)[EPC], const u32x4 v, float wgt) {
    if (DT == 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(wgt, __uint_as_float(v[q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(wgt, __uint_as_float(v[q] & 0xffff0000u), acc[2 * q + 1]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(wgt, __uint_as_float(v[q]), acc[q]);
    }
  };
  // U chunks per lane per round, every load of the round issued before its stores.  The
  // loads are unconditional, so that none waits for the one before it (a load under a
  // per-lane branch is waited for where the branch merges): a chunk past the block re-reads
  // its last chunk, and a dropped slot's expert row is read through a buffer resource at an
  // offset past its range, which returns zeros without a memory access (and is not used).
  // The range is checked dword by dword against the record count (2^31 - 1 here): every
  // expert row lies below 2^31 - 1 bytes from o (the workspace layout checks it), and the
  // dropped-slot offset has bit 31 set, so each dword of its access is past the range.
  constexpr uint32_t kNoRow = 0x80000000u;
  typedef __amdgpu_buffer_rsrc_t rsrc_t;
  const rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(ob), static_cast<short>(0),
                                                         0x7fffffff, 0x00020000);
  const int total = nt * ch;
  for (int base = t; base < total; base += 256 * U) {
    u32x4 vo[U][KT], vs[U], vx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * 256 < total ? base + u * 256 : total - 1;
      const int tl = idx / ch, c = idx - tl * ch;
      const size_t n = static_cast<size_t>(tok0 + tl);
      const char* xrow = xb + n * rowbytes + c * 16;
#pragma unroll
      for (int jj = 0; jj < KT; ++jj) {
        const int r = rows_s[tl][jj];
        const uint32_t off = r >= 0 ? static_cast<uint32_t>(r) * static_cast<uint32_t>(rowbytes) +
                                          static_cast<uint32_t>(c) * 16u
                                    : kNoRow;
        vo[u][jj] = __builtin_amdgcn_raw_buffer_load_b128(orsrc, off, 0, 2);   // nt
      }
      if (sb) vs[u] = ld_stream(reinterpret_cast<const u32x4*>(sb + n * rowbytes + c * 16));
      if (a.residual) vx[u] = ld_stream(reinterpret_cast<const u32x4*>(xrow));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * 256;
      if (idx >= total) continue;
      const int tl = idx / ch, c = idx - tl * ch;
      const size_t n = static_cast<size_t>(tok0 + tl);
      float acc[EPC];
#pragma unroll
      for (int q = 0; q < EPC; ++q) acc[q] = 0.f;
#pragma unroll
      for (int jj = 0; jj < KT; ++jj)
        if (rows_s[tl][jj] >= 0) add(acc, vo[u][jj], w_s[tl][jj]);
      if (sb) add(acc, vs[u], 1.0f);
      if (a.residual) add(acc, vx[u], 1.0f);
      u32x4 out;
      if (DT == 1) {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) out[q] = __float_as_uint(acc[q]);
      }
      st_stream(reinterpret_cast<u32x4*>(yb + n * rowbytes + c * 16), out);
    }
  }
}

__global__ __launch_bounds__(256) void aux_only_kernel(CombineArgs a) { aux_final(a); }

}  // namespace

hipError_t launch_combine(const CombineArgs& args, hipStream_t s) {
  if (args.k < 1 || args.k > kMaxTopK || args.M <= 0) return hipErrorInvalidValue;
  // One round of U chunks per lane covers the block's tokens (whole rows, at least one), and
  // a short batch still spreads over one block per CU.  Rows of up to 128 chunks take two
  // chunks per lane (more blocks), longer rows four (more loads in flight per lane).
  CombineArgs a = args;
  const int ch = a.M / (a.dtype == 1 ? 8 : 4);
  const int u = ch <= 128 ? 2 : 4;
  a.tpb = std::max(1, std::min({kTokMax, 256 * u / ch, a.N / 256}));
  const int grid = (a.N + a.tpb - 1) / a.tpb;
  if (grid == 0) return hipSuccess;
#define MOE_COMBINE_K(KV)                                                                  \
  case KV:                                                                                  \
    if (a.dtype == 1 && u == 2)                                                             \
      hipLaunchKernelGGL((combine_kernel<1, KV, 2>), dim3(grid), dim3(256), 0, s, a);      \
    else if (a.dtype == 1)                                                                  \
      hipLaunchKernelGGL((combine_kernel<1, KV, 4>), dim3(grid), dim3(256), 0, s, a);      \
    else if (u == 2)                                                                        \
      hipLaunchKernelGGL((combine_kernel<0, KV, 2>), dim3(grid), dim3(256), 0, s, a);      \
    else                                                                                    \
      hipLaunchKernelGGL((combine_kernel<0, KV, 4>), dim3(grid), dim3(256), 0, s, a);      \
    break;
  switch (a.k) {
    MOE_COMBINE_K(1) MOE_COMBINE_K(2) MOE_COMBINE_K(3) MOE_COMBINE_K(4)
    MOE_COMBINE_K(5) MOE_COMBINE_K(6) MOE_COMBINE_K(7) MOE_COMBINE_K(8)
  }
#undef MOE_COMBINE_K
  return hipGetLastError();
}

hipError_t launch_aux_only(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(aux_only_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
