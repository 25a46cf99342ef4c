// moe_gate: per-group expert capacity positions by prefix scans, and the dispatch offsets.
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
// offsets_kernel then lays the kept rows out expert-major, (expert, group, position)
// order, with the capacity padding squeezed out, and cuts each expert's rows into BM-row
// GEMM tiles ([GShard] "Sharding 与 MoE 的交替布局": group-major tokens regrouped into an
// expert-major buffer).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

// One wave per (group, expert).
__global__ __launch_bounds__(256) void gate_scan_kernel(ScanArgs a) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= a.G * a.E) return;
  const int g = gw / a.E, e = gw - g * a.E;
  const int nbg = a.nbg;

  // aux partials: sum of probabilities and of selections over the group's blocks
  const size_t pe = (static_cast<size_t>(g) * a.E + e) * nbg;
  double ps = 0.0;
  int cs = 0;
  for (int b = lane; b < nbg; b += 64) {
    ps += a.psum[pe + b];
    cs += a.sel[pe + b];
  }
  ps = wave_sum(ps);
  cs = wave_sum(cs);
  if (lane == 0) {
    a.Pg[static_cast<size_t>(g) * a.E + e] = ps;
    a.Cg[static_cast<size_t>(g) * a.E + e] = cs;
  }

  int base = 0;
  for (int j = 0; j < a.k; ++j) {
    const size_t o = ((static_cast<size_t>(g) * a.k + j) * a.E + e) * nbg;
    const int32_t* h = a.ahist + o;
    int32_t* ob = a.abase + o;
    int run = 0;
    for (int b0 = 0; b0 < nbg; b0 += 64) {
      const int b = b0 + lane;
      const int v = b < nbg ? h[b] : 0;
      const int inc = wave_inclusive_scan(v);
      if (b < nbg) ob[b] = base + run + inc - v;
      run += __shfl(inc, 63, 64);
    }
    if (lane == 0) a.ntot[(static_cast<size_t>(g) * a.k + j) * a.E + e] = run;
    base = min(a.C, base + run);
  }
  if (lane == 0) a.count[static_cast<size_t>(g) * a.E + e] = base;
}

// Exclusive scan of one value per thread over a 256-thread block; returns the total in *tot.
__device__ int block_exclusive_scan(int v, int* tot, int* scratch /* [4] */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) scratch[w] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = scratch[i];
    if (i < w) before += s;
    all += s;
  }
  __syncthreads();
  *tot = all;
  return before + inc - v;
}

__global__ __launch_bounds__(256) void offsets_kernel(OffsetsArgs a) {
  __shared__ int scratch[4];
  __shared__ int red[4];
  const int t = threadIdx.x;
  const int E = a.E, G = a.G;
  int tot_e = 0;
  if (t < E)
    for (int g = 0; g < G; ++g) tot_e += a.count[static_cast<size_t>(g) * E + t];
  int R = 0;
  const int off = block_exclusive_scan(t < E ? tot_e : 0, &R, scratch);
  if (t < E) {
    a.offset[t] = off;
    int run = off;
    for (int g = 0; g < G; ++g) {
      a.gbase[static_cast<size_t>(g) * E + t] = run;
      run += a.count[static_cast<size_t>(g) * E + t];
    }
  }
  if (t == 0) a.offset[E] = R;

  // GEMM tiles: expert e's rows [offset[e], offset[e] + tot_e) cut into BM-row pieces.
  const int mt = t < E ? (tot_e + a.BM - 1) / a.BM : 0;
  int ntiles = 0;
  const int tp = block_exclusive_scan(mt, &ntiles, scratch);
  for (int i = 0; i < mt; ++i) {
    TileDesc d;
    d.expert = t;
    d.row0 = off + i * a.BM;
    d.nrows = min(a.BM, tot_e - i * a.BM);
    d.pad = 0;
    a.tiles[tp + i] = d;
  }
  if (t == 0) *a.num_tiles = ntiles;

  // stats: R, dropped slots (active but over capacity), fully dropped (zeroed here, counted
  // by the dispatch kernel), random-routing skips (selected but not active).
  int act = 0;
  for (int i = t; i < G * a.k * E; i += 256) act += a.ntot[i];
  act = wave_sum(act);
  if ((t & 63) == 0) red[t >> 6] = act;
  __syncthreads();
  if (t == 0) {
    const int active = red[0] + red[1] + red[2] + red[3];
    a.stats[0] = R;
    a.stats[1] = active - R;
    a.stats[2] = 0;
    a.stats[3] = a.N * a.k - active;
  }
}

__global__ void empty_kernel(EmptyArgs a) {
  const int t = threadIdx.x;
  for (int i = t; i < a.G * a.E; i += blockDim.x) a.count[i] = 0;
  for (int i = t; i <= a.E; i += blockDim.x) a.offset[i] = 0;
  if (t < 4) a.stats[t] = 0;
  if (t == 0) *a.aux = 0.f;
}

}  // namespace

hipError_t launch_gate_scan(const ScanArgs& a, hipStream_t s) {
  const int waves = a.G * a.E;
  hipLaunchKernelGGL(gate_scan_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_offsets(const OffsetsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(offsets_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_empty(const EmptyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
