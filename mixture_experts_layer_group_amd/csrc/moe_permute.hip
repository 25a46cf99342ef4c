// moe_permute: dispatch offsets, capacity positions, dispatch rows, and the row scatter of x
// into the compact expert-major buffer.
//
// One block = the 64 tokens of one router block.  Every block first derives, from the kept
// counts per (group, expert), where its group's rows of each expert start in the compact
// buffer: rows are laid out expert-major, in (expert, group, position) order with the
// capacity padding squeezed out ([GShard] "Sharding 与 MoE 的交替布局": group-major tokens
// regrouped into an expert-major buffer).  Block 0 also writes the expert offsets, the list
// of BM-row GEMM tiles and the stats.
//
// For rank j, lane = token: the lanes that chose the same expert and are active are found
// with one ballot per bit of the expert id, and the count of such lanes below gives the
// in-block prefix; adding the block base from gate_scan_kernel gives the position of
// [GShard] "Top-2 gating 的四个机制 / Expert capacity" (kept iff < C).  The row is the
// (group, expert) base plus the position.  A token whose slots are all lost passes through
// the residual ([GShard] "Capacity overflow 会跳过 expert computation"), counted in stats[2].
//
// The scatter then copies every kept token's row of x once per kept slot, 16 bytes per
// lane, reading x once ([GShard] "Automatic propagation 与 manual override": dispatch as an
// index tensor plus a gather, here the transposed scatter).  A router block's rows are cut
// into `slices` column slices, one block each, so that enough blocks are in flight to
// cover HBM latency; the slices repeat the (cheap) position work and slice 0 alone writes
// the per-slot outputs.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

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

// Row bases of group g's experts in the compact buffer (into gbase_s), and in block 0 the
// expert offsets, the GEMM tile list and the stats.  T threads share an expert's sum over
// the groups (T = 256 / E rounded down to a power of two, at most 64).
__device__ void offsets(const PermuteArgs& a, int g, int* gbase_s, int* scratch) {
  const int t = threadIdx.x, E = a.E, G = a.G;
  int T = 64;
  while (T * E > 256) T >>= 1;
  const int e = t / T, sub = t - e * T;
  const bool lead = sub == 0 && e < E;
  int tot = 0, pre = 0;
  if (e < E)
    for (int gg = sub; gg < G; gg += T) {
      const int c = a.count[static_cast<size_t>(gg) * E + e];
      tot += c;
      if (gg < g) pre += c;
    }
  for (int o = T >> 1; o > 0; o >>= 1) {  // lanes e*T .. e*T+T-1 sit in one wave
    tot += __shfl_xor(tot, o, 64);
    pre += __shfl_xor(pre, o, 64);
  }
  int R = 0;
  const int off = block_exclusive_scan(lead ? tot : 0, &R, scratch);
  if (lead) gbase_s[e] = off + pre;
  if (blockIdx.x != 0) return;

  if (lead) a.offset[e] = off;
  if (t == 0) a.offset[E] = R;
  // GEMM tiles: expert e's rows [offset[e], offset[e] + tot) cut into BM-row pieces.
  const int mt = lead ? (tot + a.BM - 1) / a.BM : 0;
  int ntiles = 0;
  const int tp = block_exclusive_scan(mt, &ntiles, scratch);
  for (int i = 0; i < mt; ++i) {
    TileDesc d;
    d.expert = e;
    d.row0 = off + i * a.BM;
    d.nrows = min(a.BM, tot - i * a.BM);
    d.pad = 0;
    a.tiles[tp + i] = d;
  }
  if (t == 0) *a.num_tiles = ntiles;
  // stats: R, dropped slots (active but over capacity), fully dropped tokens (stats[2],
  // counted below by every block), random-routing skips (selected but not active).
  int act = 0;
  for (int i = t; i < G * a.k * E; i += 256) act += a.ntot[i];
  int all = 0;
  block_exclusive_scan(act, &all, scratch);
  if (t == 0) {
    a.stats[0] = R;
    a.stats[1] = all - R;
    a.stats[3] = a.N * a.k - all;
  }
}

__global__ __launch_bounds__(256) void permute_kernel(PermuteArgs a) {
  __shared__ int rows_s[kRouteTokens][kMaxTopK];
  __shared__ float w_s[kRouteTokens][kMaxTopK];   // gate weight of each kept slot
  __shared__ int kept_any[kRouteTokens];
  __shared__ int gbase_s[kMaxExperts];
  __shared__ int scratch[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int b = blockIdx.x / a.slices, slice = blockIdx.x - b * a.slices;
  const bool meta = slice == 0;
  const int g = b / a.nbg, bi = b - g * a.nbg;
  const int tok0 = g * a.S + bi * kRouteTokens;
  const int nt = min(kRouteTokens, a.S - bi * kRouteTokens);
  const int k = a.k;
  if (t < kRouteTokens) kept_any[t] = 0;
  offsets(a, g, gbase_s, scratch);
  __syncthreads();

  const bool valid = lane < nt;
  const int n = tok0 + lane;
  for (int j = w; j < k; j += 4) {
    const size_t o = static_cast<size_t>(n) * k + j;
    const int e = valid ? a.topk_idx[o] : 0;
    const bool act = valid && a.active[o] != 0;
    uint64_t m = ballot(act);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bb = ballot(on);
      m &= on ? bb : ~bb;
    }
    const int prefix = __popcll(m & lanes_below());
    if (valid) {
      int p = a.C;
      if (act) p = a.abase[((static_cast<size_t>(g) * k + j) * a.E + e) * a.nbg + bi] + prefix;
      const bool kept = act && p < a.C;
      const int r = kept ? gbase_s[e] + p : -1;
      // kept slots' weights are final (the meta slice zeroes the others only)
      const float wk = kept ? a.topk_w[o] : 0.f;
      if (meta) {
        a.pos[o] = kept ? p : -1;
        a.row[o] = r;
        if (!kept) a.topk_w[o] = 0.f;
        if (kept && a.tok_of_row) a.tok_of_row[r] = n;
        if (kept && a.w_of_row) a.w_of_row[r] = wk;
      }
      rows_s[lane][j] = r;
      w_s[lane][j] = wk;
      if (kept) kept_any[lane] = 1;
    }
  }
  __syncthreads();
  if (w == 0 && meta) {
    const bool dropped = valid && kept_any[lane] == 0;
    const int c = __popcll(ballot(dropped));
    if (lane == 0 && c) atomicAdd(&a.stats[2], c);
  }
  if (!a.x) return;

  const int esz = a.dtype == 1 ? 2 : 4;
  const int chr = a.M * esz / 16;  // 16-byte chunks per row
  const int per = (chr + a.slices - 1) / a.slices;
  const int c0 = slice * per;
  const int ch = max(0, min(chr, c0 + per) - c0);  // chunks of this slice
  const size_t rowbytes = static_cast<size_t>(a.M) * esz;
  const char* __restrict__ xb = static_cast<const char*>(a.x) + c0 * 16;
  char* __restrict__ bb = static_cast<char*>(a.buf) + c0 * 16;
  // U chunks per thread per round: all U loads are issued before any store, so U loads are
  // in flight per lane (the stores may not be reordered above loads the compiler cannot
  // prove disjoint from them).  With dy, the same chunk of dy is scaled by each kept slot's
  // weight into dout (fp32 product, rounded like every stored value).
  constexpr int U = 4;
  const bool wdy = a.dy != nullptr;
  const char* __restrict__ yb = wdy ? static_cast<const char*>(a.dy) + c0 * 16 : nullptr;
  char* __restrict__ ob = wdy ? static_cast<char*>(a.dout) + c0 * 16 : nullptr;
  const int total = nt * ch;
  for (int base = t; base < total; base += 256 * U) {
    u32x4 v[U], yv[U];
    int tlv[U], cv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = base + u * 256;
      tlv[u] = -1;
      if (idx < total) {
        const int tl = idx / ch, c = idx - tl * ch;
        if (kept_any[tl]) {
          tlv[u] = tl;
          cv[u] = c;
          const size_t off = static_cast<size_t>(tok0 + tl) * rowbytes + c * 16;
          v[u] = *reinterpret_cast<const u32x4*>(xb + off);
          if (wdy) yv[u] = *reinterpret_cast<const u32x4*>(yb + off);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tlv[u] < 0) continue;
      for (int j = 0; j < k; ++j) {
        const int r = rows_s[tlv[u]][j];
        if (r < 0) continue;
        const size_t off = static_cast<size_t>(r) * rowbytes + cv[u] * 16;
        *reinterpret_cast<u32x4*>(bb + off) = v[u];
        if (wdy) {
          const float w = w_s[tlv[u]][j];
          u32x4 sv;
          if (a.dtype == 1) {
#pragma unroll
            for (int x = 0; x < 4; ++x)
              sv[x] = pack_bf16x2(w * __builtin_bit_cast(float, yv[u][x] << 16),
                                  w * __builtin_bit_cast(float, yv[u][x] & 0xffff0000u));
          } else {   // 4 fp32 values, scaled as a vector
            const f32x4 yf = __builtin_bit_cast(f32x4, yv[u]);
            sv = __builtin_bit_cast(u32x4, yf * w);
          }
          *reinterpret_cast<u32x4*>(ob + off) = sv;
        }
      }
    }
  }
}

}  // namespace

int permute_slices(const PermuteArgs& a) {
  const int blocks = a.G * a.nbg;
  const int chr = a.M * (a.dtype == 1 ? 2 : 4) / 16;
  int slices = 1;
  if (a.x)
    while (blocks * slices < 2048 && chr / (2 * slices) >= 16) slices *= 2;
  return slices;
}

hipError_t launch_permute(const PermuteArgs& a0, hipStream_t s) {
  PermuteArgs a = a0;
  a.slices = permute_slices(a);
  const int64_t grid = static_cast<int64_t>(a.G) * a.nbg * a.slices;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
