// Index arithmetic of the expert GEMM launches: which output tile a block computes, and the
// batched GEMM entries of the backward pass.  Plain integer code with no HIP dependency, so
// that the kernels (device) and a host-side check compiled with a plain C++ compiler use the
// same functions.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MOE_HD __host__ __device__
#else
#define MOE_HD
#endif

namespace moe {

struct TileDesc {         // one BM-row tile of one expert in the compact buffer
  int32_t expert, row0, nrows, pad;
};

// One entry of a batched GEMM problem: element offsets of its A, B and C blocks and its K
// depth (0 writes a zero block).
struct BatchEntry {
  int64_t a_off, b_off, c_off;
  int32_t K, pad;
};

// The tiles of one launch: problem 0 has mt0 x nt0 tiles (mt0 of a routed problem is the
// device tile count), problem 1 mt1 x nt1 (0 x 0 when the launch has one problem).
// tpe > 0: both problems are batched with tpe tiles per entry, and the entries are dealt over
// the XCD ranges (see tile_coord).  plain: 0, or the order of a one-problem launch that is not
// dealt: 1 plain block order, 2 expert-synchronous (see tile_coord).
struct TileSpace {
  int mt0, nt0, mt1, nt1, tpe, plain;
};

struct TileCoord {
  int prob, mt, nt;       // problem, m-tile and n-tile of the block
};

MOE_HD inline int tile_total(const TileSpace& s) { return s.mt0 * s.nt0 + s.mt1 * s.nt1; }

// nprob: problems in the launch (1 or 2; with 1, mt1 = nt1 = 0); batched: every problem of the
// launch is batched; mpe0 / mpe1: m-tiles per entry.  Entries are dealt only when every entry
// of both problems has the same number of tiles and they tile the launch exactly.  plain (1 or
// 2) applies to one-problem launches that are not dealt; 2 needs a multiple of 8 n-tiles and
// falls back to the XCD ranges otherwise.
MOE_HD inline TileSpace tile_space(int mt0, int nt0, int mt1, int nt1, int nprob, bool batched,
                                   int mpe0, int mpe1, int plain = 0) {
  TileSpace s{mt0, nt0, nprob > 1 ? mt1 : 0, nprob > 1 ? nt1 : 0, 0, 0};
  if (batched) {
    const int tpe = mpe0 * nt0;
    const bool same = nprob == 1 || mpe1 * nt1 == tpe;
    const int total = tile_total(s);
    const int T = tpe > 0 ? total / tpe : 0;
    if (same && T > 0 && T * tpe == total) s.tpe = tpe;
  }
  s.plain = s.tpe == 0 && s.mt1 * s.nt1 == 0 && (plain == 1 || (plain == 2 && (nt0 & 7) == 0))
                ? plain : 0;
  return s;
}

// Block bid -> tile, or false past the last tile.
//  * Blocks are dispatched round-robin over the 8 XCDs (block b runs on XCD b % 8); each XCD
//    receives a contiguous range of tile slots, so neighbouring tiles share its L2.
//  * Dealt batched launches (the weight gradients: one entry per expert or token range, each
//    with its own K, which a skewed router makes very unequal): slot s lies in bin b (bins of
//    ceil((T - b) / 8) slots laid out in order, T entries) and holds entry 8 (s - start of bin
//    b) + b, so each XCD range gets every 8th entry rather than 8 neighbouring ones and an
//    entry's tiles stay together.
//  * Other two-problem launches (routed experts + shared experts, whose K can differ): each
//    XCD range holds its eighth of problem 0's tiles, then its eighth of problem 1's, so
//    every XCD gets the same share of both.  Problem 1's remainder tiles go to the XCDs
//    after those that took problem 0's remainder (cyclically), which keeps each XCD's tile
//    count equal to the number of blocks it receives.
//  * Plain order (block b takes slot b) for launches whose row operand does not fit the
//    last-level cache while the weights are shared: consecutive slots go to the 8 XCDs in
//    turn, so the XCDs work on the same expert at the same time and share its weight tiles
//    through that cache, and each XCD keeps whole m-tiles (all their n-tiles at once) in its
//    L2, reading every row once.
//  * Expert-synchronous order for launches whose weights do not fit the last-level cache
//    while the rows do: XCD x takes n-tiles [x nb, (x + 1) nb) (nb = n-tiles / 8) of every
//    m-tile, m-tiles in list order, so all XCDs work on the same expert at the same time and
//    that expert's weights (each n-range read by one XCD) and rows stay in that cache until
//    the next expert; group_m m-tiles sweep the XCD's nb n-tiles.
//  * Inside a problem, group_m m-tiles sweep the n-tiles together (L2 reuse of the weight
//    tiles across an expert's row tiles and of the row tiles across n-tiles).
// A bijection from [0, tile_total) onto the tiles of both problems.
MOE_HD inline bool tile_coord(const TileSpace& s, int bid, int group_m, TileCoord& c) {
  const int tot0 = s.mt0 * s.nt0, total = tile_total(s), tot1 = total - tot0;
  if (bid < 0 || bid >= total) return false;
  const int xcd = bid & 7, loc = bid >> 3, q = total >> 3, r = total & 7;
  if (s.plain == 2) {
    const int nb = s.nt0 >> 3;   // every XCD holds mt0 nb tiles: total / 8 exactly
    const int per_group = group_m * nb;
    const int grp = loc / per_group, first = grp * group_m;
    const int gsz = s.mt0 - first < group_m ? s.mt0 - first : group_m;
    const int in = loc - grp * per_group;
    c.prob = 0;
    c.mt = first + in % gsz;
    c.nt = xcd * nb + in / gsz;
    return true;
  }
  int pid = s.plain ? bid : xcd * q + (xcd < r ? xcd : r) + loc;
  if (s.tpe == 0 && tot0 > 0 && tot1 > 0) {
    const int q0 = tot0 >> 3, r0 = tot0 & 7, q1 = tot1 >> 3, r1 = tot1 & 7;
    const int n0 = q0 + (xcd < r0 ? 1 : 0);   // problem 0 tiles of this XCD
    if (loc < n0) {
      pid = xcd * q0 + (xcd < r0 ? xcd : r0) + loc;
    } else {
      int before = 0;   // XCDs below this one that take one of problem 1's remainder tiles
      for (int x = 0; x < xcd; ++x) before += ((x - r0 + 8) & 7) < r1 ? 1 : 0;
      pid = tot0 + xcd * q1 + before + (loc - n0);
    }
  }
  if (s.tpe > 0) {
    const int T = total / s.tpe;
    const int sl = pid / s.tpe, rr = pid - sl * s.tpe;
    int b = 0, base = 0;
    while (b < 7 && base + ((T - b + 7) >> 3) <= sl) {
      base += (T - b + 7) >> 3;
      ++b;
    }
    pid = (8 * (sl - base) + b) * s.tpe + rr;
  }
  const bool second = pid >= tot0;
  const int lp = second ? pid - tot0 : pid;
  const int mts = second ? s.mt1 : s.mt0;
  const int nts = second ? s.nt1 : s.nt0;
  const int per_group = group_m * nts;
  const int grp = lp / per_group;
  const int first = grp * group_m;
  const int gsz = mts - first < group_m ? mts - first : group_m;
  const int in = lp - grp * per_group;
  c.prob = second ? 1 : 0;
  c.mt = first + in % gsz;
  c.nt = in / gsz;
  return true;
}

// m-tile mt of a batched problem whose entries have `rows` rows each: its entry, first row and
// row count.
MOE_HD inline void batch_tile(int mt, int rows, int BM, int& entry, int& row0, int& nrows) {
  const int mpe = (rows + BM - 1) / BM;
  entry = mt / mpe;
  row0 = (mt - entry * mpe) * BM;
  nrows = rows - row0 < BM ? rows - row0 : BM;
}

// ---- batched entries of the backward's GEMMs (element offsets; operands read in place)

// Routed expert e, whose kept rows are [o, o + cnt) of the compact buffers:
//   dW2_e [M, H] = dout_e^T h_e       (A = dout [R, M], B = h [R, H], C = dW2 [E + Es, M, H])
//   dW1_e [H1, M] = dz1_e^T buf_e     (A = dz1 [R, H1], B = buf [R, M], C = dW1 [E + Es, H1, M])
MOE_HD inline BatchEntry dw2_routed_entry(int e, int64_t o, int cnt, int64_t M, int64_t H) {
  return BatchEntry{o * M, o * H, e * M * H, cnt, 0};
}
MOE_HD inline BatchEntry dw1_routed_entry(int e, int64_t o, int cnt, int64_t M, int64_t H1) {
  return BatchEntry{o * H1, o * M, e * H1 * M, cnt, 0};
}
// Shared expert q's dz over every token: (dy W2_{E+q}) act'(z), K = M, output columns q H1 of
// dz1sh [N, Es H1] (A = dy [N, M], B = W2 [E + Es, M, H] read K-major).
MOE_HD inline BatchEntry dhsh_entry(int q, int E, int64_t M, int64_t H, int64_t H1) {
  return BatchEntry{0, (E + q) * M * H, q * H1, static_cast<int32_t>(M), 0};
}
// Shared expert q over token range sr (tokens [sr kshared, +kshared) of N), into fp32 partial
// i = q nshared + sr:
//   dy_s^T hsh_q,s    (A = dy [N, M], B = hsh [N, Es H], C = partials [Es nshared, M, H])
//   dz1sh_q,s^T x_s   (A = dz1sh [N, Es H1], B = x [N, M], C = partials [Es nshared, H1, M])
MOE_HD inline int shared_range_rows(int sr, int64_t kshared, int64_t N) {
  const int64_t n0 = sr * kshared;
  return static_cast<int>(kshared < N - n0 ? kshared : N - n0);
}
MOE_HD inline BatchEntry dw2_shared_entry(int q, int sr, int nshared, int64_t kshared, int64_t N,
                                          int Es, int64_t M, int64_t H) {
  const int64_t n0 = sr * kshared, i = static_cast<int64_t>(q) * nshared + sr;
  return BatchEntry{n0 * M, n0 * Es * H + q * H, i * M * H, shared_range_rows(sr, kshared, N), 0};
}
MOE_HD inline BatchEntry dw1_shared_entry(int q, int sr, int nshared, int64_t kshared, int64_t N,
                                          int Es, int64_t M, int64_t H1) {
  const int64_t n0 = sr * kshared, i = static_cast<int64_t>(q) * nshared + sr;
  return BatchEntry{n0 * Es * H1 + q * H1, n0 * M, i * H1 * M, shared_range_rows(sr, kshared, N),
                    0};
}
// Router weight gradient over token range q: dl_q^T x_q [E, M] into fp32 partial q
// (A = dlp [N, Ep], B = x [N, M], C = partials [nsplit, E, M]).
MOE_HD inline BatchEntry dwg_entry(int q, int64_t ksplit, int64_t N, int64_t Ep, int64_t M,
                                   int64_t E) {
  const int64_t n0 = q * ksplit;
  return BatchEntry{n0 * Ep, n0 * M, q * E * M,
                    static_cast<int32_t>(ksplit < N - n0 ? ksplit : N - n0), 0};
}

}  // namespace moe
