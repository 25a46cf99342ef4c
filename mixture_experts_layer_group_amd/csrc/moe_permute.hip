// moe_permute: capacity positions, dispatch rows, and the row scatter of x into the compact
// expert-major buffer.
//
// One block = the 64 tokens of one router block.  For rank j, lane = token: the lanes that
// chose the same expert and are active are found with one ballot per bit of the expert id,
// and the count of such lanes below gives the in-block prefix; adding the block base from
// gate_scan_kernel gives the position of [GShard] "Top-2 gating 的四个机制 / Expert
// capacity" (kept iff < C).  The row is the (group, expert) base of offsets_kernel plus the
// position.  A token whose slots are all lost passes through the residual ([GShard]
// "Capacity overflow 会跳过 expert computation"), counted in stats[2].
//
// The scatter then copies every kept token's row of x once per kept slot, 16 bytes per
// lane, reading x once ([GShard] "Automatic propagation 与 manual override": dispatch as an
// index tensor plus a gather, here the transposed scatter).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void permute_kernel(PermuteArgs a) {
  __shared__ int rows_s[kRouteTokens][kMaxTopK];
  __shared__ int kept_any[kRouteTokens];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int b = blockIdx.x;
  const int g = b / a.nbg, bi = b - g * a.nbg;
  const int tok0 = g * a.S + bi * kRouteTokens;
  const int nt = min(kRouteTokens, a.S - bi * kRouteTokens);
  const int k = a.k;
  if (t < kRouteTokens) kept_any[t] = 0;
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
      const int r = kept ? a.gbase[static_cast<size_t>(g) * a.E + e] + p : -1;
      a.pos[o] = kept ? p : -1;
      a.row[o] = r;
      if (!kept) a.topk_w[o] = 0.f;
      rows_s[lane][j] = r;
      if (kept) kept_any[lane] = 1;
    }
  }
  __syncthreads();
  if (w == 0) {
    const bool dropped = valid && kept_any[lane] == 0;
    const int c = __popcll(ballot(dropped));
    if (lane == 0 && c) atomicAdd(&a.stats[2], c);
  }
  if (!a.x) return;

  const int esz = a.dtype == 1 ? 2 : 4;
  const int ch = a.M * esz / 16;  // 16-byte chunks per row
  const size_t rowbytes = static_cast<size_t>(a.M) * esz;
  const char* xb = static_cast<const char*>(a.x);
  char* bb = static_cast<char*>(a.buf);
  for (int idx = t; idx < nt * ch; idx += 256) {
    const int tl = idx / ch, c = idx - tl * ch;
    if (!kept_any[tl]) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(xb + static_cast<size_t>(tok0 + tl) * rowbytes + c * 16);
    for (int j = 0; j < k; ++j) {
      const int r = rows_s[tl][j];
      if (r >= 0) *reinterpret_cast<u32x4*>(bb + static_cast<size_t>(r) * rowbytes + c * 16) = v;
    }
  }
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int grid = a.G * a.nbg;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(permute_kernel, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
