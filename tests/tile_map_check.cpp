// Host-side check of the expert GEMM's tile order and of the backward's batched GEMM entries
// (mixture_experts_layer_group_amd/csrc/moe_tile_map.h, the same functions the kernels call).
//
// For random layer shapes it rebuilds, on the host, every launch of the expert GEMM that the
// forward and backward passes make (problem sizes, tile lists, batched entries) and checks:
//   * tile_coord is a bijection from [0, total) onto the tiles of the launch's problems;
//   * every decoded tile lies inside its problem (m-tile < m-tiles, n-tile < n-tiles) and a
//     batched tile's entry index inside its own problem's entry array;
//   * the elements that the tile's A, B and C (and, for the fused activation gradient, z)
//     blocks cover stay inside that problem's buffers;
//   * the C blocks of different entries of one batched problem do not overlap.
// Prints "ok <shapes> <launches> <tiles>" and exits 0, or prints the first failure and exits 1.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "moe_tile_map.h"

using moe::BatchEntry;

namespace {

constexpr int kGroupM = 8;
// m-tile group of the shape's routed launches: one expert's largest m-tile count, at most
// kGroupM (the launcher's rule); batched and dense launches keep kGroupM
int g_group_m = kGroupM;
// tile shape of the launches being checked: 256 x 256 (bf16 kernel) or 64 x 64 (fp32 kernel);
// a gated GEMM 1 writes half the columns it computes
int kBM = 256, kBN = 256;

struct Problem {
  std::string name;
  // routed: tile list (m-tiles) over the compact rows; batched: entries; else dense rows
  std::vector<moe::TileDesc> tiles;
  std::vector<BatchEntry> entries;
  bool routed = false, batched = false;
  int plain = 0;           // one-problem launch order: 1 plain, 2 expert-synchronous
  int64_t rows = 0;        // dense: rows; batched: rows of every entry
  int64_t N = 0, K = 0;    // output columns, depth (dense / routed; entries carry their own)
  int64_t lda = 0, ldb = 0, ldc = 0, b_stride = 0;
  bool akm = false, bkm = false;
  int glu_h = 0;           // gated output (C also receives columns + glu_h)
  bool gated_b = false;    // gated B: the tile's gate rows plus their up rows glu_h later
  bool gather = false;     // A rows come through a row -> token index (any row < a_elems/lda)
  int64_t kseg = 0, seg_stride = 0;   // row-major B split along K into segments (0: none)
  int64_t a_elems = 0, b_elems = 0, c_elems = 0;
  int bn = kBN;            // output columns per tile
};

int fails = 0;
long long n_tiles_checked = 0;

bool fail(const std::string& what) {
  if (fails++ < 5) std::printf("FAIL %s\n", what.c_str());
  return false;
}

bool check_range(const Problem& p, const char* op, int64_t lo, int64_t hi, int64_t n,
                 const char* ctx) {
  if (lo < 0 || hi > n) {
    char b[512];
    std::snprintf(b, sizeof b, "%s: %s covers [%lld, %lld) of %lld elements (%s)", p.name.c_str(),
                  op, (long long)lo, (long long)hi, (long long)n, ctx);
    return fail(b);
  }
  return true;
}

// One tile: the element ranges of its operand blocks.
bool check_tile(const Problem& p, int mt, int nt) {
  int64_t row0, nrows, K = p.K, aoff = 0, boff = 0, coff = 0, e = 0;
  char ctx[128];
  std::snprintf(ctx, sizeof ctx, "m-tile %d n-tile %d", mt, nt);
  if (p.routed) {
    if (mt >= (int)p.tiles.size()) return fail(p.name + ": m-tile past the tile list");
    row0 = p.tiles[mt].row0;
    nrows = p.tiles[mt].nrows;
    e = p.tiles[mt].expert;
  } else if (p.batched) {
    int be, r0, nr;
    moe::batch_tile(mt, (int)p.rows, kBM, be, r0, nr);
    if (be < 0 || be >= (int)p.entries.size()) return fail(p.name + ": entry index past the array");
    const BatchEntry& d = p.entries[be];
    row0 = r0; nrows = nr; K = d.K; aoff = d.a_off; boff = d.b_off; coff = d.c_off;
  } else {
    row0 = int64_t(mt) * kBM;
    nrows = std::min<int64_t>(kBM, p.rows - row0);
  }
  const int64_t c0 = int64_t(nt) * p.bn, ncols = std::min<int64_t>(p.bn, p.N - c0);
  if (nrows <= 0 || ncols <= 0 || K < 0) return fail(p.name + ": empty tile " + ctx);
  bool ok = true;
  if (K > 0) {
    if (p.gather) {
      // rows are gathered through an index whose values the dispatch bounds by the token
      // count; the whole A range is readable
    } else if (p.akm) {
      ok &= check_range(p, "A", aoff + row0, aoff + (K - 1) * p.lda + row0 + nrows, p.a_elems, ctx);
    } else {
      // with a K-major B the K loop runs whole chunks (64 deep, 16 in the fp32 kernel), and a
      // row-major A row is read to the end of its last chunk
      const int64_t bk = kBM == 256 ? 64 : 16;
      const int64_t KA = p.bkm ? (K + bk - 1) / bk * bk : K;
      ok &= check_range(p, "A", aoff + row0 * p.lda, aoff + (row0 + nrows - 1) * p.lda + KA,
                        p.a_elems, ctx);
    }
    const int64_t bb = e * p.b_stride + boff;
    if (p.bkm) {
      ok &= check_range(p, "B", bb + c0, bb + (K - 1) * p.ldb + c0 + ncols, p.b_elems, ctx);
    } else if (p.gated_b) {
      // output column c reads gate row (c / H) 2H + c % H and that row + H
      const int64_t H = p.glu_h;
      const int64_t first = (c0 / H) * 2 * H + c0 % H;
      const int64_t lastc = c0 + ncols - 1;
      const int64_t last = (lastc / H) * 2 * H + lastc % H + H;
      ok &= check_range(p, "B", bb + first * p.ldb, bb + last * p.ldb + K, p.b_elems, ctx);
    } else if (p.kseg > 0 && K > p.kseg) {
      // K element kk of row c sits at (kk / kseg) seg_stride + c ldb + kk % kseg
      const int64_t nseg = (K + p.kseg - 1) / p.kseg;
      ok &= check_range(p, "B", bb + c0 * p.ldb,
                        bb + (nseg - 1) * p.seg_stride + (c0 + ncols - 1) * p.ldb + p.kseg,
                        p.b_elems, ctx);
    } else {
      ok &= check_range(p, "B", bb + c0 * p.ldb, bb + (c0 + ncols - 1) * p.ldb + K, p.b_elems,
                        ctx);
    }
  }
  const int64_t cend = coff + (row0 + nrows - 1) * p.ldc + c0 + ncols + (p.glu_h && !p.gated_b ? p.glu_h : 0);
  ok &= check_range(p, "C", coff + row0 * p.ldc + c0, cend, p.c_elems, ctx);
  ++n_tiles_checked;
  return ok;
}

int m_tiles(const Problem& p) {
  if (p.routed) return (int)p.tiles.size();
  if (p.batched) return (int)p.entries.size() * (int)((p.rows + kBM - 1) / kBM);
  return (int)((p.rows + kBM - 1) / kBM);
}

// Distinct entries of a batched problem write disjoint C blocks: rows x [c_off, c_off + ...).
bool check_disjoint(const Problem& p) {
  if (!p.batched) return true;
  std::vector<std::pair<int64_t, int64_t>> iv;
  for (const BatchEntry& d : p.entries) {
    // a C block is rows x (columns of the output, + glu_h for gated dz) at pitch ldc; blocks
    // of one problem either start a whole block apart (row-stacked) or interleave by columns
    const int64_t width = p.N + (p.glu_h && !p.gated_b ? p.glu_h : 0);
    if (d.c_off % p.ldc + width <= p.ldc)   // column band [c_off % ldc, + width) of rows
      iv.push_back({d.c_off, d.c_off + (p.rows - 1) * p.ldc + width});
    else
      return fail(p.name + ": entry C block wraps past its row");
  }
  // column-interleaved blocks (same rows, distinct column bands) or row-stacked blocks
  for (size_t i = 0; i < iv.size(); ++i) {
    const int64_t start = iv[i].first;
    const int64_t row_start = start / p.ldc, col = start % p.ldc;
    const int64_t width = p.N + (p.glu_h && !p.gated_b ? p.glu_h : 0);
    for (size_t j = 0; j < i; ++j) {
      const int64_t s2 = iv[j].first, r2 = s2 / p.ldc, c2 = s2 % p.ldc;
      const bool rows_overlap = !(row_start + p.rows <= r2 || r2 + p.rows <= row_start);
      const bool cols_overlap = !(col + width <= c2 || c2 + width <= col);
      if (rows_overlap && cols_overlap) return fail(p.name + ": two entries write one C element");
    }
  }
  return true;
}

// One launch of one or two problems: bijection and per-tile checks.
bool check_launch(const Problem& p0, const Problem* p1) {
  const int nprob = p1 ? 2 : 1;
  const int mt0 = m_tiles(p0), nt0 = (int)((p0.N + p0.bn - 1) / p0.bn);
  const int mt1 = p1 ? m_tiles(*p1) : 0, nt1 = p1 ? (int)((p1->N + p1->bn - 1) / p1->bn) : 0;
  const bool batched = p0.batched && (!p1 || p1->batched);
  const int mpe0 = (int)((p0.rows + kBM - 1) / kBM);
  const int mpe1 = p1 ? (int)((p1->rows + kBM - 1) / kBM) : 0;
  const moe::TileSpace sp = moe::tile_space(mt0, nt0, mt1, nt1, nprob, batched, mpe0, mpe1,
                                            p0.plain);
  const int total = moe::tile_total(sp);
  const int gm = p0.routed ? g_group_m : kGroupM;
  // the grid the host launches covers the problems' tile bounds
  std::vector<char> seen((size_t)total, 0);
  bool ok = true;
  moe::TileCoord c;
  int per_xcd[8][2] = {};
  for (int bid = 0; bid < total; ++bid) {
    if (!moe::tile_coord(sp, bid, gm, c)) return fail(p0.name + ": block inside the grid decoded as none");
    if (c.prob == 0 || c.prob == 1) per_xcd[bid & 7][c.prob]++;
    const Problem& P = c.prob ? *p1 : p0;
    const int mts = c.prob ? mt1 : mt0, nts = c.prob ? nt1 : nt0;
    if (c.prob < 0 || c.prob >= nprob || c.mt < 0 || c.mt >= mts || c.nt < 0 || c.nt >= nts)
      return fail(P.name + ": decoded tile outside its problem");
    const size_t lin = (size_t)(c.prob ? mt0 * nt0 : 0) + (size_t)c.mt * nts + c.nt;
    if (seen[lin]++) return fail(P.name + ": two blocks decode to one tile");
    ok &= check_tile(P, c.mt, c.nt);
  }
  if (moe::tile_coord(sp, total, gm, c)) return fail(p0.name + ": block past the grid decoded");
  // two problems that are not dealt by entries: every XCD (blocks bid with equal bid % 8)
  // holds an eighth of each problem's tiles, rounded down or up
  if (p1 && sp.tpe == 0) {
    const int tot[2] = {mt0 * nt0, mt1 * nt1};
    for (int x = 0; x < 8; ++x)
      for (int q = 0; q < 2; ++q)
        if (per_xcd[x][q] != tot[q] / 8 && per_xcd[x][q] != (tot[q] + 7) / 8)
          return fail(p0.name + ": an XCD's share of a problem's tiles is unbalanced");
  }
  ok &= check_disjoint(p0);
  if (p1) ok &= check_disjoint(*p1);
  return ok;
}

struct Shape {
  int64_t N, G, M, H, E, Es, k, C;
  bool glu;
  bool f32;   // fp32 layer: 64 x 64 tiles
};

// Every expert GEMM launch of the forward and the backward for one shape and one routing
// outcome (kept rows per expert cnt[e]).
int check_shape(const Shape& s, const std::vector<int>& cnt) {
  const int64_t N = s.N, M = s.M, H = s.H, E = s.E, Es = s.Es, k = s.k;
  const int64_t H1 = s.glu ? 2 * H : H;
  const int64_t S = N / s.G;
  const int64_t Rmax = std::min<int64_t>(k * N, s.G * E * std::min<int64_t>(s.C, S));
  const int64_t ra = Rmax + kBM;   // rows allocated in the compact buffers
  std::vector<int64_t> off(E + 1, 0);
  for (int e = 0; e < E; ++e) off[e + 1] = off[e] + cnt[e];
  const int64_t R = off[E];
  if (R > Rmax) return fail("routing keeps more rows than Rmax"), 0;
  {
    const int64_t maxr = std::min<int64_t>(N, s.G * std::min<int64_t>(s.C, S));
    const int64_t mt = (maxr + kBM - 1) / kBM;
    g_group_m = (int)std::max<int64_t>(1, std::min<int64_t>(kGroupM, mt));
    for (int e = 0; e < E; ++e)
      if ((cnt[e] + kBM - 1) / kBM > mt) return fail("an expert holds more m-tiles than the bound"), 0;
  }
  // device tile list: expert e's rows cut into BM-row pieces, in expert order
  std::vector<moe::TileDesc> tiles;
  for (int e = 0; e < E; ++e)
    for (int64_t i = 0; i * kBM < cnt[e]; ++i)
      tiles.push_back({e, (int32_t)(off[e] + i * kBM), (int32_t)std::min<int64_t>(kBM, cnt[e] - i * kBM), 0});
  const int64_t max_tiles = Rmax / kBM + E + 1;
  if ((int64_t)tiles.size() > max_tiles) return fail("tile list longer than its bound"), 0;
  int launches = 0;

  // ---- forward GEMM 1: h = act(x[tok] W1_e^T) (+ shared: h_sh = act(x W1_sh^T))
  Problem g1;
  g1.name = "fwd GEMM 1";
  g1.routed = true; g1.tiles = tiles; g1.gather = true;
  // the launcher's rule: no shared experts and the weights of min(E, 8) experts (one per
  // XCD under the XCD ranges) larger than 256 MB
  g1.plain = Es == 0 &&
                     std::min<int64_t>(E, 8) * H1 * M * (kBM == 256 ? 2 : 4) > (int64_t(256) << 20)
                 ? 2 : 0;
  g1.N = H; g1.K = M; g1.lda = M; g1.ldb = M; g1.ldc = H; g1.b_stride = H1 * M;
  g1.gated_b = s.glu; g1.glu_h = s.glu ? (int)H : 0;
  g1.a_elems = N * M; g1.b_elems = (E + Es) * H1 * M; g1.c_elems = ra * H;
  g1.bn = s.glu ? kBN / 2 : kBN;
  Problem g1s = g1;
  g1s.name = "fwd GEMM 1 shared";
  g1s.routed = false; g1s.tiles.clear(); g1s.gather = false; g1s.rows = N;
  g1s.N = Es * H; g1s.ldc = Es * H; g1s.b_stride = 0; g1s.c_elems = N * Es * H;
  g1s.b_elems = Es * H1 * M;   // B based at the first shared expert
  if (!check_launch(g1, Es ? &g1s : nullptr)) return 0;
  ++launches;
  // ---- forward GEMM 2: o = h W2_e^T (+ shared: o_sh = h_sh [W2_sh..]^T over K segments)
  Problem g2;
  g2.name = "fwd GEMM 2";
  // the launcher's rule: no shared experts and h larger than 256 MB
  g2.plain = Es == 0 && Rmax * H * (kBM == 256 ? 2 : 4) > (int64_t(256) << 20) ? 1 : 0;
  g2.routed = true; g2.tiles = tiles;
  g2.N = M; g2.K = H; g2.lda = H; g2.ldb = H; g2.ldc = M; g2.b_stride = M * H;
  g2.a_elems = ra * H; g2.b_elems = (E + Es) * M * H; g2.c_elems = ra * M;
  Problem g2s;
  g2s.name = "fwd GEMM 2 shared";
  g2s.rows = N; g2s.N = M; g2s.K = Es * H; g2s.lda = Es * H; g2s.ldb = H; g2s.ldc = M;
  g2s.a_elems = N * Es * H; g2s.c_elems = N * M;
  // the K axis runs over the shared experts' W2 blocks: segments of H, M H apart
  g2s.kseg = H; g2s.seg_stride = M * H; g2s.b_elems = Es * M * H;
  if (!check_launch(g2, Es ? &g2s : nullptr)) return 0;
  ++launches;

  // ---- backward
  const int64_t Ep = (E + 63) / 64 * 64;
  const int64_t tilesg = ((E + 255) / 256) * ((M + 255) / 256);
  const int64_t Npad = (N + 127) / 128 * 128;
  const int64_t Ssp = std::max<int64_t>(1, std::min<int64_t>((256 + tilesg - 1) / tilesg, Npad / 128));
  const int64_t ksplit = std::max<int64_t>(128, (Npad / Ssp + 127) / 128 * 128);
  const int64_t nsplit = (N + ksplit - 1) / ksplit;
  const int64_t avg = (N * k + E - 1) / E;
  int64_t kshared = std::max<int64_t>(512, (avg + 127) / 128 * 128);
  kshared = std::max<int64_t>(kshared, (N + 31) / 32);
  const int64_t nshared = Es ? (N + kshared - 1) / kshared : 0;

  std::vector<BatchEntry> e2(E + Es * nshared), e1(E + Es * nshared), eh(Es), eg(nsplit);
  for (int e = 0; e < E; ++e) {
    e2[e] = moe::dw2_routed_entry(e, off[e], cnt[e], M, H);
    e1[e] = moe::dw1_routed_entry(e, off[e], cnt[e], M, H1);
  }
  for (int q = 0; q < Es; ++q) eh[q] = moe::dhsh_entry(q, (int)E, M, H, H1);
  for (int i = 0; i < Es * nshared; ++i) {
    const int q = i / (int)nshared, sr = i - q * (int)nshared;
    e2[E + i] = moe::dw2_shared_entry(q, sr, (int)nshared, kshared, N, (int)Es, M, H);
    e1[E + i] = moe::dw1_shared_entry(q, sr, (int)nshared, kshared, N, (int)Es, M, H1);
  }
  for (int q = 0; q < nsplit; ++q) eg[q] = moe::dwg_entry(q, ksplit, N, Ep, M, E);
  int64_t shared_rows = 0;
  for (int sr = 0; sr < nshared; ++sr) shared_rows += moe::shared_range_rows(sr, kshared, N);
  if (Es && shared_rows != N) return fail("shared token ranges do not cover the tokens"), 0;
  int64_t split_rows = 0;
  for (const BatchEntry& d : eg) split_rows += d.K;
  if (split_rows != N) return fail("router weight-gradient ranges do not cover the tokens"), 0;

  // z1 / h recompute: as forward GEMM 1 but A = buf (compact rows), output H1 columns
  Problem z1 = g1;
  z1.name = "bwd z1";
  z1.gather = false; z1.a_elems = ra * M; z1.N = H1; z1.ldc = H1; z1.c_elems = ra * H1;
  z1.gated_b = false; z1.glu_h = 0; z1.bn = kBN;
  Problem z1s = g1s;
  z1s.name = "bwd z1 shared";
  z1s.N = Es * H1; z1s.ldc = Es * H1; z1s.c_elems = N * Es * H1; z1s.gated_b = false;
  z1s.glu_h = 0; z1s.bn = kBN;
  if (!check_launch(z1, Es ? &z1s : nullptr)) return 0;
  ++launches;
  // dz: routed (dy rows gathered, W2 K-major) + shared dz (batched dhsh entries)
  Problem dz;
  dz.name = "bwd dz";
  dz.routed = true; dz.tiles = tiles; dz.gather = true;
  dz.N = H; dz.K = M; dz.lda = M; dz.ldb = H; dz.ldc = H1; dz.b_stride = M * H; dz.bkm = true;
  dz.glu_h = s.glu ? (int)H : 0;
  dz.a_elems = N * M; dz.b_elems = (E + Es) * M * H; dz.c_elems = ra * H1;
  Problem dzs;
  dzs.name = "bwd dz shared";
  dzs.batched = true; dzs.entries = eh; dzs.rows = N;
  dzs.N = H; dzs.lda = M; dzs.ldb = H; dzs.ldc = Es * H1; dzs.bkm = true;
  dzs.glu_h = s.glu ? (int)H : 0;
  dzs.a_elems = N * M; dzs.b_elems = (E + Es) * M * H; dzs.c_elems = N * Es * H1;
  if (!check_launch(dz, Es ? &dzs : nullptr)) return 0;
  ++launches;
  // dx rows: dz W1_e (K-major W1), shared dz_sh W1_sh over k = (q, h')
  Problem dx;
  dx.name = "bwd dx";
  dx.routed = true; dx.tiles = tiles;
  dx.N = M; dx.K = H1; dx.lda = H1; dx.ldb = M; dx.ldc = M; dx.b_stride = H1 * M; dx.bkm = true;
  dx.a_elems = ra * H1; dx.b_elems = (E + Es) * H1 * M; dx.c_elems = ra * M;
  Problem dxs;
  dxs.name = "bwd dx shared";
  dxs.rows = N; dxs.N = M; dxs.K = Es * H1; dxs.lda = Es * H1; dxs.ldb = M; dxs.ldc = M;
  dxs.bkm = true; dxs.a_elems = N * Es * H1; dxs.b_elems = Es * H1 * M; dxs.c_elems = N * M;
  // router dx term: dlp [N, Ep] (row-major, K = E of its Ep columns) x Wg [E, M] read K-major;
  // the dx launch's second problem when there are no shared experts
  Problem rt;
  rt.name = "bwd router dx";
  rt.rows = N; rt.N = M; rt.K = E; rt.lda = Ep; rt.ldb = M; rt.ldc = M; rt.bkm = true;
  rt.a_elems = N * Ep; rt.b_elems = E * M; rt.c_elems = N * M;
  if (!check_launch(dx, Es ? &dxs : &rt)) return 0;
  ++launches;
  if (Es) {
    if (!check_launch(rt, nullptr)) return 0;
    ++launches;
  }
  // dWg partials
  Problem wg;
  wg.name = "bwd dWg";
  wg.batched = true; wg.entries = eg; wg.rows = E;
  wg.N = M; wg.lda = Ep; wg.ldb = M; wg.ldc = M; wg.akm = wg.bkm = true;
  wg.a_elems = N * Ep; wg.b_elems = N * M; wg.c_elems = nsplit * E * M;
  if (!check_launch(wg, nullptr)) return 0;
  ++launches;
  // dW2: routed entries + shared token ranges
  Problem w2;
  w2.name = "bwd dW2";
  w2.batched = true; w2.entries.assign(e2.begin(), e2.begin() + E); w2.rows = M;
  w2.N = H; w2.lda = M; w2.ldb = H; w2.ldc = H; w2.akm = w2.bkm = true;
  w2.a_elems = ra * M; w2.b_elems = ra * H; w2.c_elems = (E + Es) * M * H;
  Problem w2s;
  w2s.name = "bwd dW2 shared";
  w2s.batched = true; w2s.entries.assign(e2.begin() + E, e2.end()); w2s.rows = M;
  w2s.N = H; w2s.lda = M; w2s.ldb = Es * H; w2s.ldc = H; w2s.akm = w2s.bkm = true;
  w2s.a_elems = N * M; w2s.b_elems = N * Es * H; w2s.c_elems = Es * nshared * M * H;
  if (!check_launch(w2, Es ? &w2s : nullptr)) return 0;
  ++launches;
  // dW1: routed entries + shared token ranges
  Problem w1;
  w1.name = "bwd dW1";
  w1.batched = true; w1.entries.assign(e1.begin(), e1.begin() + E); w1.rows = H1;
  w1.N = M; w1.lda = H1; w1.ldb = M; w1.ldc = M; w1.akm = w1.bkm = true;
  w1.a_elems = ra * H1; w1.b_elems = ra * M; w1.c_elems = (E + Es) * H1 * M;
  Problem w1s;
  w1s.name = "bwd dW1 shared";
  w1s.batched = true; w1s.entries.assign(e1.begin() + E, e1.end()); w1s.rows = H1;
  w1s.N = M; w1s.lda = Es * H1; w1s.ldb = M; w1s.ldc = M; w1s.akm = w1s.bkm = true;
  w1s.a_elems = N * Es * H1; w1s.b_elems = N * M; w1s.c_elems = Es * nshared * H1 * M;
  if (!check_launch(w1, Es ? &w1s : nullptr)) return 0;
  ++launches;
  return launches;
}

// Kept rows per expert: a random split of R <= Rmax over the experts, skewed toward low
// expert indices half of the time, with empty experts, each expert bounded by G min(C, S).
std::vector<int> random_counts(std::mt19937_64& rng, const Shape& s) {
  const int64_t S = s.N / s.G, cap = s.G * std::min<int64_t>(s.C, S);
  const int64_t Rmax = std::min<int64_t>(s.k * s.N, s.E * cap);
  std::uniform_real_distribution<double> U(0.0, 1.0);
  int64_t R = (int64_t)(U(rng) * (Rmax + 1));
  if (R > Rmax) R = Rmax;
  if (rng() % 4 == 0) R = Rmax;
  std::vector<double> w(s.E);
  const bool skew = rng() % 2;
  for (int e = 0; e < s.E; ++e) w[e] = (skew ? 1.0 / (e + 1) : 1.0) * (rng() % 5 == 0 ? 0.0 : U(rng));
  std::vector<int> cnt(s.E, 0);
  int64_t left = R;
  // fill by weighted draws in blocks, respecting the per-expert cap
  double ws = 0;
  for (double v : w) ws += v;
  if (ws <= 0) { w.assign(s.E, 1.0); ws = s.E; }
  for (int e = 0; e < s.E && left > 0; ++e) {
    int64_t c = (int64_t)(R * w[e] / ws);
    c = std::min<int64_t>({c, cap, left});
    cnt[e] = (int)c;
    left -= c;
  }
  for (int e = 0; left > 0; e = (e + 1) % s.E) {   // the remainder, round-robin under the cap
    const int64_t c = std::min<int64_t>(cap - cnt[e], left);
    cnt[e] += (int)c;
    left -= c;
  }
  return cnt;
}

}  // namespace

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 10000;
  std::mt19937_64 rng(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
  int shapes = 0, launches = 0, two = 0;
  // fixed shapes first: the reference workloads (G, N, M, H, E, Es, k, C, gated)
  const Shape fixed[] = {
      {256, 1, 64, 128, 4, 0, 2, 128, false, true},
      {16384, 8, 1024, 4096, 64, 0, 2, 64, false, false},
      {32768, 1, 768, 3072, 128, 0, 1, 320, false, false},
      {16384, 1, 4096, 14336, 8, 0, 2, 16384, false, false},
      {32768, 1, 2048, 1408, 64, 2, 6, 4608, false, false},
      {32768, 1, 2048, 1408, 64, 2, 6, 4608, true, false},
      {16384, 1, 2048, 512, 256, 1, 8, 640, true, false},
  };
  for (int i = 0; i < n && !fails; ++i) {
    Shape s;
    if (i < (int)(sizeof fixed / sizeof fixed[0])) {
      s = fixed[i];
    } else {
      std::uniform_int_distribution<int> d(0, 1 << 30);
      s.G = 1 + d(rng) % 8;
      s.N = s.G * (1 + d(rng) % (i % 10 == 0 ? 8192 : 1024));
      s.M = 128 * (1 + d(rng) % 16);
      s.H = 128 * (1 + d(rng) % 16);
      s.E = 1 + d(rng) % (i % 7 == 0 ? 256 : 40);
      s.Es = d(rng) % 3 == 0 ? 1 + d(rng) % 3 : 0;
      s.k = 1 + d(rng) % std::min<int64_t>(8, s.E);
      s.C = 1 + d(rng) % (s.N / s.G + 8);
      s.glu = d(rng) % 3 == 0;
      s.f32 = d(rng) % 4 == 0;
      if (s.f32) {   // the fp32 kernel's shapes: M, H multiples of 64
        s.M = 64 * (1 + d(rng) % 16);
        s.H = 64 * (1 + d(rng) % 16);
      }
    }
    kBM = kBN = s.f32 ? 64 : 256;
    const std::vector<int> cnt = random_counts(rng, s);
    const int l = check_shape(s, cnt);
    if (!l) {
      std::printf("  at shape N=%lld G=%lld M=%lld H=%lld E=%lld Es=%lld k=%lld C=%lld glu=%d "
                  "f32=%d\n", (long long)s.N, (long long)s.G, (long long)s.M, (long long)s.H,
                  (long long)s.E, (long long)s.Es, (long long)s.k, (long long)s.C, (int)s.glu,
                  (int)s.f32);
      return 1;
    }
    launches += l;
    two += s.Es ? 1 : 0;
    ++shapes;
  }
  if (fails) return 1;
  std::printf("ok %d shapes (%d with shared experts) %d launches %lld tiles\n", shapes, two,
              launches, n_tiles_checked);
  return 0;
}
