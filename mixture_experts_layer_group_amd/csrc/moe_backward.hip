// moe_backward: the kernels of the layer's backward pass besides the expert GEMMs.
//
// The loss is L = sum_n <dy_n, y_n> + a_aux aux + a_z z_loss + a_dev dev_loss.  Routing
// decisions (top-k, group limits, random routing, capacity) are piecewise constant and carry
// no gradient ([MegaBlocks] "3. 负载均衡损失": the balance loss reaches the router only
// through the scores, the token counts being constants).  The expert part runs the chain rule
// backwards through combine, GEMM 2, the activation and GEMM 1 ([GShard] "MoE Transformer":
// the expert FFN; [Lec16] "DeepSeek V3 MoE (670B)": the gated form); the router part through
// the gate normalisation, the softmax and the balance and z losses.  Every reduction runs in
// a fixed order, so the results are bitwise deterministic.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

template <int DT>
__device__ __forceinline__ void st_elem(void* p, int64_t i, float v) {
  if (DT == 1)
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else
    static_cast<float*>(p)[i] = v;
}

// 16-byte vectors of the layer dtype: 8 bf16 or 4 fp32 values.
template <int DT>
struct Vec {
  static constexpr int N = DT == 1 ? 8 : 4;
  float v[N];
  __device__ __forceinline__ void load(const void* p, int64_t i) {  // i: element index
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p) + i * (DT == 1 ? 2 : 4));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (DT == 1) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      } else {
        v[q] = __uint_as_float(w[q]);
      }
    }
  }
  __device__ __forceinline__ void store(void* p, int64_t i) const {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = DT == 1 ? pack_bf16x2(v[2 * q], v[2 * q + 1]) : __float_as_uint(v[q]);
    *reinterpret_cast<u32x4*>(static_cast<char*>(p) + i * (DT == 1 ? 2 : 4)) = w;
  }
};

// One block: the batched GEMM entries of the weight gradients, which read the compact
// buffers, x and dl in place as K-major operands (K = rows of the expert, or tokens).
//   dW2_e [M, H]  = dout_e^T h_e        dW1_e [H1, M] = dz1_e^T buf_e
//   shared q, token range s (fp32 partials):  dy_s^T hsh_q,s    dz1sh_q,s^T x_s
//   dWg token range s [E, M] = dl_s^T x_s (fp32 partials)
// and of the shared experts' dz_q = (dy W2_{E+q}) act'(z_q) (K-major weights, output columns
// q H1 of dz1sh).
__global__ __launch_bounds__(256) void bwd_setup_kernel(BwdSetupArgs a) {
  const int t = threadIdx.x, E = a.E;
  for (int e = t; e < E; e += 256) {
    const int64_t o = a.offset[e];
    const int cnt = a.offset[e + 1] - a.offset[e];
    a.dw2[e] = dw2_routed_entry(e, o, cnt, a.M, a.H);
    a.dw1[e] = dw1_routed_entry(e, o, cnt, a.M, a.H1);
  }
  for (int q = t; q < a.Es; q += 256)  // shared experts' dz over every token
    a.dhsh[q] = dhsh_entry(q, E, a.M, a.H, a.H1);
  // shared experts' weight gradients over token range s (rows s * kshared ..) into fp32
  // partials [q][s], summed in range order afterwards
  for (int i = t; i < a.Es * a.nshared; i += 256) {
    const int q = i / a.nshared, sr = i - q * a.nshared;
    a.dw2[E + i] = dw2_shared_entry(q, sr, a.nshared, a.kshared, a.N, a.Es, a.M, a.H);
    a.dw1[E + i] = dw1_shared_entry(q, sr, a.nshared, a.kshared, a.N, a.Es, a.M, a.H1);
  }
  for (int q = t; q < a.nsplit; q += 256)  // dWg [E, M] over token range q
    a.dwg[q] = dwg_entry(q, a.ksplit, a.N, a.Ep, a.M, E);
}

// Router backward, one wave per token: dL/dp through the gate normalisation (none, sum or
// p-norm of the selected probabilities), the balance losses (counts are constants), the
// softmax, and the z-loss: dl_e = p_e (dp_e - sum_i p_i dp_i) + a_z 2 lse p_e / N.
__global__ __launch_bounds__(256) void router_bwd_kernel(RouterBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= a.N) return;
  const int E = a.E, k = a.k;
  const float* l = a.logits + static_cast<int64_t>(n) * E;
  float mx = -INFINITY;
  for (int e = lane; e < E; e += 64) mx = fmaxf(mx, l[e]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float se = 0.0f;
  for (int e = lane; e < E; e += 64) se += expf(l[e] - mx);
  se = wave_sum(se);
  const float lse = mx + logf(se);

  // gradient of the selected probabilities through the normalisation: with w_j = ps_j / D,
  // D = (sum_i ps_i^P)^(1/P) (sum: P = 1), dps_i = (dw_i - w_i^(P-1) sum_j w_j dw_j) / D.
  // Written this way the two terms cancel exactly where the weights do not depend on the
  // logits; a single selected expert under either normalisation has weight 1 whatever the
  // logits, so it passes no gradient at all (the difference of two separately rounded
  // quotients would leak dw's size times the rounding into dl).
  float dps[kMaxTopK];
  int sel[kMaxTopK];
  {
    float ps[kMaxTopK], dw[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      sel[j] = -1;
      ps[j] = dw[j] = dps[j] = 0.0f;
      if (j < k) {
        sel[j] = a.topk_idx[static_cast<int64_t>(n) * k + j];
        ps[j] = expf(l[sel[j]] - mx) / se;
        dw[j] = a.dw[static_cast<int64_t>(n) * k + j];
      }
    }
    if (a.norm == 0) {
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) dps[j] = dw[j];
    } else if (k > 1) {
      const float P = a.norm == 1 ? 1.0f : a.norm_p;
      float D = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) D += a.norm == 1 ? ps[j] : powf(ps[j], P);
      if (a.norm == 2) D = powf(D, 1.0f / P);
      float w[kMaxTopK], t = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        w[j] = j < k ? ps[j] / D : 0.0f;
        t = fmaf(w[j], dw[j], t);
      }
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) dps[j] = (dw[j] - (a.norm == 1 ? t : powf(w[j], P - 1.0f) * t)) / D;
    }
  }
  const int g = n / a.S;
  const float inv_gs = 1.0f / (static_cast<float>(a.G) * a.S);
  const int gs = E / a.n_eg;
  float pe[4], dp[4];
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    pe[i] = dp[i] = 0.0f;
    if (e < E) {
      pe[i] = expf(l[e] - mx) / se;
      float d = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k && sel[j] == e) d += dps[j];
      const float c_e = static_cast<float>(a.Cg[static_cast<int64_t>(g) * E + e]);
      d += a.coef_aux * E * c_e * inv_gs / (static_cast<float>(k) * a.S);
      if (a.coef_dev != 0.0f) {  // f_j = mean over the expert group of E c / (k S)
        const int j0 = (e / gs) * gs;
        float cs = 0.0f;
        for (int x = 0; x < gs; ++x) cs += static_cast<float>(a.Cg[static_cast<int64_t>(g) * E + j0 + x]);
        d += a.coef_dev * (E * cs / (gs * static_cast<float>(k) * a.S)) * inv_gs;
      }
      dp[i] = d;
      acc = fmaf(pe[i], d, acc);
    }
  }
  const float sp = wave_sum(acc);
  const float zc = a.coef_z * 2.0f * lse / static_cast<float>(a.N);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    if (e < E) a.dl[static_cast<int64_t>(n) * E + e] = pe[i] * (dp[i] - sp) + zc * pe[i];
  }
}

// dbg partial sums: block ch sums dl over its 256 tokens (in order) for every expert.
__global__ __launch_bounds__(256) void dbg_partial_kernel(DwgArgs a) {
  // block (chunk of 256 tokens, 64 experts); wave w sums tokens [64 w, 64 w + 64) of the chunk
  // for expert e = 64 eb + lane, then the 4 wave sums are added in wave order
  __shared__ float part[4][64];
  const int ch = blockIdx.x, eb = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = eb * 64 + lane;
  const int n0 = ch * 256 + w * 64, nn = max(0, min(64, a.N - n0));
  float sb = 0.0f;
  if (e < a.E) {
    const float* p = a.dl + static_cast<int64_t>(n0) * a.E + e;
    int r = 0;
    for (; r + 8 <= nn; r += 8) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = p[static_cast<int64_t>(r + i) * a.E];
#pragma unroll
      for (int i = 0; i < 8; ++i) sb += v[i];
    }
    for (; r < nn; ++r) sb += p[static_cast<int64_t>(r) * a.E];
  }
  part[w][lane] = sb;
  __syncthreads();
  if (w == 0 && e < a.E)
    a.partb[static_cast<int64_t>(ch) * a.E + e] = ((part[0][lane] + part[1][lane]) + part[2][lane]) +
                                                   part[3][lane];
}

// Combine weights' gradient from the dgrad GEMM's per-n-tile partial dot products.
__global__ __launch_bounds__(256) void dw_reduce_kernel(const int32_t* __restrict__ row,
                                                        const float* __restrict__ dwp,
                                                        float* __restrict__ dw, int64_t n,
                                                        int ntn) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const int r = row[i];
  float s = 0.f;
  if (r >= 0)
    for (int t = 0; t < ntn; ++t) s += dwp[static_cast<int64_t>(r) * ntn + t];
  dw[i] = s;
}

// out = sum of S fp32 partial arrays in order, 4 elements per thread.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           float* __restrict__ out, int64_t n,
                                                           int S) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  // partials 1 .. S-1 added in order, their loads issued 8 at a time
  int q = 1;
  for (; q + 8 <= S; q += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = *reinterpret_cast<const f32x4*>(part + static_cast<int64_t>(q + u) * n + i);
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int x = 0; x < 4; ++x) acc[x] += v[u][x];
  }
  for (; q < S; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + static_cast<int64_t>(q) * n + i);
#pragma unroll
    for (int x = 0; x < 4; ++x) acc[x] += v[x];
  }
  *reinterpret_cast<f32x4*>(out + i) = acc;
}

// dbg = sum of the chunk partials in order.
__global__ __launch_bounds__(256) void dbg_reduce_kernel(DwgArgs a) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.E) return;
  float s = 0.0f;
  int ch = 0;
  for (; ch + 8 <= a.nchunks; ch += 8) {   // in order, loads issued 8 at a time
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = a.partb[static_cast<int64_t>(ch + u) * a.E + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; ch < a.nchunks; ++ch) s += a.partb[static_cast<int64_t>(ch) * a.E + e];
  a.dbg[e] = s;
}

// dx_n = [res] dy_n + sum_j dx_rows[row_nj] + dx_shared_n + (dl Wg)_n, summed in that order
// in fp32; the router term comes from a GEMM (dxrt).  One wave per token, 16 bytes per lane.
template <int DT>
__global__ __launch_bounds__(256) void dx_final_kernel(DxArgs a) {
  constexpr int V = Vec<DT>::N;
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= a.N) return;
  int rows[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    rows[j] = j < a.k ? a.row[static_cast<int64_t>(n) * a.k + j] : -1;
  const int64_t base = static_cast<int64_t>(n) * a.M;
  for (int m = lane * V; m < a.M; m += 64 * V) {
    Vec<DT> acc, t;
#pragma unroll
    for (int x = 0; x < V; ++x) acc.v[x] = 0.0f;
    if (a.residual) acc.load(a.dy, base + m);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (rows[j] < 0) continue;
      t.load(a.dxr, static_cast<int64_t>(rows[j]) * a.M + m);
#pragma unroll
      for (int x = 0; x < V; ++x) acc.v[x] += t.v[x];
    }
    if (a.dxsh) {
      t.load(a.dxsh, base + m);
#pragma unroll
      for (int x = 0; x < V; ++x) acc.v[x] += t.v[x];
    }
    t.load(a.dxrt, base + m);
#pragma unroll
    for (int x = 0; x < V; ++x) acc.v[x] += t.v[x];
    acc.store(a.dx, base + m);
  }
}

// The router's dgrad operand dlp [N, Ep] = dl in the layer dtype, zero beyond E (Ep = E
// rounded up to 64), the A operand of dxrt = dl Wg (Wg itself is read in place as a K-major
// operand) and of dWg = dl^T x.
template <int DT>
__global__ __launch_bounds__(256) void router_dgrad_prep_kernel(RouterPrepArgs a) {
  const int64_t nd = static_cast<int64_t>(a.N) * a.Ep;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < nd;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / a.Ep;
    const int e = static_cast<int>(i - r * a.Ep);
    st_elem<DT>(a.dlp, i, e < a.E ? a.dl[r * a.E + e] : 0.0f);
  }
}

__global__ void zero_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0.0f;
}

int grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return static_cast<int>(b < 1 ? 1 : (b > 65535 ? 65535 : b));
}

}  // namespace

hipError_t launch_bwd_setup(const BwdSetupArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bwd_setup_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const RouterBwdArgs& a, hipStream_t s) {
  const int grid = (a.N + 3) / 4;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(router_bwd_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dbg(const DwgArgs& a, hipStream_t s) {
  if (a.nchunks == 0 || !a.dbg) return hipSuccess;
  hipLaunchKernelGGL(dbg_partial_kernel, dim3(a.nchunks, (a.E + 63) / 64), dim3(256), 0, s, a);
  hipLaunchKernelGGL(dbg_reduce_kernel, dim3((a.E + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dw_reduce(const int32_t* row, const float* dwp, float* dw, int64_t n, int ntn,
                            hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dw_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     s, row, dwp, dw, n, ntn);
  return hipGetLastError();
}

hipError_t launch_split_reduce(const float* part, float* out, int64_t n, int S, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int64_t grid = (n / 4 + 255) / 256;
  hipLaunchKernelGGL(split_reduce_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s,
                     part, out, n, S);
  return hipGetLastError();
}

hipError_t launch_router_dgrad_prep(const RouterPrepArgs& a, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(a.N) * a.Ep;
  if (a.dtype == 1)
    hipLaunchKernelGGL(router_dgrad_prep_kernel<1>, dim3(grid_for(n)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(router_dgrad_prep_kernel<0>, dim3(grid_for(n)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dx_final(const DxArgs& a, hipStream_t s) {
  const int grid = (a.N + 3) / 4;
  if (grid == 0) return hipSuccess;
  if (a.dtype == 1)
    hipLaunchKernelGGL(dx_final_kernel<1>, dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(dx_final_kernel<0>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace moe
