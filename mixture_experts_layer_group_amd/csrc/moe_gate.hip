// moe_gate: per-group expert capacity positions by prefix scans.
//
// [GShard] "Top-2 gating 的四个机制 / Expert capacity" and "Local group dispatching": each of
// the G groups routes on its own and an expert takes at most C tokens per group; a slot
// beyond capacity is not computed.  Positions are assigned rank-major (all 1st choices in
// token order, then all 2nd choices, ...).  As a scan this is, per (group, expert):
//   pos(n, j) = base_j + (active rank-j slots of the expert before n in the group),
//   kept iff pos < C,   base_0 = 0,   base_{j+1} = min(C, base_j + n_j),
// where n_j counts the group's active rank-j slots of the expert.  The router left one
// histogram per 64-token block; gate_scan_kernel scans those per (group, rank, expert) to
// give every block its base, and moe_permute adds the in-block prefix.
//
// One block per (group, expert), one wave per rank j: every wave loads its rank's block
// histogram and its share of the blocks' probability sums and selection counts (up to 512
// blocks of each at once, so the loads overlap), the k totals n_j meet in LDS, and each wave
// then runs the base recurrence over the ranks below it and writes its scan.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kChunks = 8;                 // 64-block chunks loaded together per wave
constexpr int kPass = kChunks * kWave;     // router blocks per pass

__global__ __launch_bounds__(kMaxTopK * kWave) void gate_scan_kernel(ScanArgs a) {
  __shared__ int tot_s[kMaxTopK];
  __shared__ double ps_s[kMaxTopK];
  __shared__ int cs_s[kMaxTopK];
  const int lane = threadIdx.x & 63;
  const int j = threadIdx.x >> 6;  // rank of this wave
  const int k = a.k, E = a.E, nbg = a.nbg;
  const int g = blockIdx.x / E, e = blockIdx.x - g * E;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.stats[2] = 0;  // counted by the dispatch kernel

  // aux partials: probabilities and selections over the group's blocks, split over the waves,
  // and n_j: active rank-j slots of the expert in the group.  Each round issues all of its
  // loads (kChunks of each array per lane) before the first is used; the sums run in block
  // order per lane as before.
  const size_t pe = (static_cast<size_t>(g) * E + e) * nbg;
  const size_t o = ((static_cast<size_t>(g) * k + j) * E + e) * nbg;
  const int32_t* __restrict__ h = a.ahist + o;
  const int stride = k * kWave;
  double ps = 0.0;
  int cs = 0;
  int v[kChunks];
  int tot = 0;
  for (int b0 = 0, p0 = threadIdx.x; b0 < nbg || p0 < nbg; b0 += kPass, p0 += kChunks * stride) {
    double pv[kChunks];
    int sv[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int b = b0 + c * kWave + lane;
      v[c] = b < nbg ? h[b] : 0;
      const int bp = p0 + c * stride;
      pv[c] = bp < nbg ? a.psum[pe + bp] : 0.0;
      sv[c] = bp < nbg ? a.sel[pe + bp] : 0;
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      tot += v[c];
      ps += pv[c];
      cs += sv[c];
    }
  }
  ps = wave_sum(ps);
  cs = wave_sum(cs);
  tot = wave_sum(tot);
  if (lane == 0) {
    tot_s[j] = tot;
    ps_s[j] = ps;
    cs_s[j] = cs;
  }
  __syncthreads();

  int base = 0;
  for (int i = 0; i < j; ++i) base = min(a.C, base + tot_s[i]);
  if (lane == 0) {
    a.ntot[(static_cast<size_t>(g) * k + j) * E + e] = tot;
    if (j == k - 1) a.count[static_cast<size_t>(g) * E + e] = min(a.C, base + tot);
    if (j == 0) {
      double P = 0.0;
      int Cs = 0;
      for (int i = 0; i < k; ++i) {
        P += ps_s[i];
        Cs += cs_s[i];
      }
      a.Pg[static_cast<size_t>(g) * E + e] = P;
      a.Cg[static_cast<size_t>(g) * E + e] = Cs;
    }
  }

  // block bases: base_j + active rank-j slots in earlier blocks
  int32_t* __restrict__ ob = a.abase + o;
  int run = base;
  for (int b0 = 0; b0 < nbg; b0 += kPass) {
    if (nbg > kPass) {  // more than one pass: the registers hold the last pass only
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int b = b0 + c * kWave + lane;
        v[c] = b < nbg ? h[b] : 0;
      }
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int b = b0 + c * kWave + lane;
      const int inc = wave_inclusive_scan(v[c]);
      if (b < nbg) ob[b] = run + inc - v[c];
      run += __shfl(inc, 63, 64);
    }
  }
}

__global__ void empty_kernel(EmptyArgs a) {
  const int t = threadIdx.x;
  for (int i = t; i < a.G * a.E; i += blockDim.x) a.count[i] = 0;
  for (int i = t; i <= a.E; i += blockDim.x) a.offset[i] = 0;
  if (t < 4) a.stats[t] = 0;
  if (t == 0) {
    if (a.aux) *a.aux = 0.f;
    if (a.z_loss) *a.z_loss = 0.f;
    if (a.dev_loss) *a.dev_loss = 0.f;
  }
}

}  // namespace

hipError_t launch_gate_scan(const ScanArgs& a, hipStream_t s) {
  const int blocks = a.G * a.E;
  hipLaunchKernelGGL(gate_scan_kernel, dim3(blocks), dim3(a.k * kWave), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_empty(const EmptyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
