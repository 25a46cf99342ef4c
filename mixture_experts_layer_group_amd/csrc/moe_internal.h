// Kernel argument blocks and launchers of the MoE layer (host <-> kernel interface).
// Nothing here is part of the public C ABI (include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_tile_map.h"

struct moe_cfg;
struct moe_meta;

namespace moe {

constexpr int kRouteTokens = 64;  // tokens per router / dispatch block (one wave of lanes)
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;
constexpr int kMaxExpertGroups = 32;  // group-limited routing: one bit per group in a lane

// Router GEMM + softmax + top-k + gates + random routing + per-block histograms.
// Blocks never straddle a group: block b covers tokens [g*S + bi*64, min(+64, (g+1)*S)),
// g = b / nbg, bi = b % nbg.
struct RouterArgs {
  const void* x;          // [N, M] T          (unused when logits_in != nullptr)
  const void* Wg;         // [E, M] T
  const float* bg;        // [E] or nullptr
  const float* u;         // [N] or nullptr
  const float* logits_in; // [N, E]: route from these logits instead of running the GEMM
  float* logits_out;      // [N, E] or nullptr
  int32_t* topk_idx;      // [N, k]
  float* topk_w;          // [N, k]  pre-drop weights (zeroed later for dropped slots)
  uint8_t* active;        // [N, k]  slot dispatched (random routing), before capacity
  double* psum;           // [G][E][nbg]  sum of softmax probabilities of the block's tokens
  int32_t* sel;           // [G][E][nbg]  top-k selections of the block's tokens
  int32_t* ahist;         // [G][k][E][nbg] active slots per rank
  double* zpart;          // [G * nbg] sum over the block's tokens of logsumexp(logits)^2
  float norm_p;           // P of the p-norm gate normalisation (norm == 2)
  int n_eg, topk_eg;      // expert groups and groups kept per token (n_eg == 1: no limit)
  int N, G, S, M, E, k, norm, rr, nbg, dtype;
};

// Per (group, expert), one wave per rank: exclusive scans over router blocks -> block bases of the capacity
// positions, kept counts, active totals, and the aux partial sums.
struct ScanArgs {
  const int32_t* ahist;   // [G][k][E][nbg]
  const double* psum;     // [G][E][nbg]
  const int32_t* sel;     // [G][E][nbg]
  int32_t* abase;         // [G][k][E][nbg]  base_j(e) + active slots in earlier blocks
  int32_t* count;         // [G, E]  kept slots (meta)
  int32_t* ntot;          // [G][k][E] active slots per rank
  double* Pg;             // [G][E]  sum_n p[n, e] over the group
  int32_t* Cg;            // [G][E]  selections over the group
  int32_t* stats;         // [4] (meta): stats[2] zeroed here for the dispatch kernel's count
  int G, E, k, C, nbg;
};

// Offsets, capacity positions, dispatch rows, dropped-weight zeroing and the row scatter
// of x.  Every block derives its group's row bases from count; block 0 writes offset,
// the tile list and stats[0,1,3].
struct PermuteArgs {
  const void* x;          // [N, M] T (nullptr: positions only)
  const int32_t* topk_idx;
  const uint8_t* active;
  const int32_t* abase;
  const int32_t* count;   // [G, E] kept slots
  const int32_t* ntot;    // [G][k][E] active slots per rank
  int32_t* offset;        // [E+1] (meta)
  TileDesc* tiles;        // [max tiles]
  int32_t* num_tiles;     // [1]
  int32_t* pos;           // [N, k] (meta)
  int32_t* row;           // [N, k] (meta)
  float* topk_w;          // [N, k] (meta): zeroed where the slot is not kept
  int32_t* stats;         // [4] (meta); stats[2] += fully dropped tokens of the block
  int32_t* tok_of_row;    // [R] token of every compact row (nullptr: not written)
  void* buf;              // [R, M] T compact expert-major rows (written iff x != nullptr)
  // backward: dout[row] = w dy[n] for every kept slot, and w_of_row[row] = w (both nullable;
  // dout needs x)
  const void* dy;
  void* dout;
  float* w_of_row;
  int N, G, S, M, E, k, C, nbg, dtype, BM;
  int slices;             // column slices per router block (set by the launcher)
};

// Activation codes of a GEMM problem (the first three are moe_cfg's act values).
constexpr int kActRelu = 0, kActGelu = 1, kActSwiglu = 2, kActNone = -1;

// One GEMM problem of the expert FFN: C[rows, N] = act(A[rows, K] . B_e[N, K]^T).
// B_e = B + e * b_stride; the K axis of B may be split into segments of kseg elements that
// sit seg_stride elements apart (the shared experts' W2 blocks).
// Gated problems (act == kActSwiglu): output column c of width N is
// Swish(A . Bg_c) * (A . Bu_c), with gate row Bg_c = B_e row (c / glu_h) 2 glu_h + c % glu_h
// and up row Bu_c = that row + glu_h (each expert's W1 stacks H gate rows on H up rows).
struct GemmProblem {
  const void* A; int64_t lda;
  const void* B; int64_t ldb; int64_t b_stride; int64_t kseg; int64_t seg_stride;
  void* C; int64_t ldc;
  int N, K;
  int a_rows;             // rows readable through A (loads clamp to a_rows - 1)
  int act;                // kAct*
  const TileDesc* tiles;  // routed: device tile list (nullptr: dense problem)
  const int32_t* num_tiles;
  int max_tiles;          // routed: grid bound on the tile count; dense: ceil(rows / BM)
  int dense_rows;         // dense problem: number of rows; batched: rows of every entry
  int glu_h;              // gated problems: hidden width H of one expert (else unused)
  const BatchEntry* batch;  // batched problem (tiles == nullptr): device entries; max_tiles =
                            // entries * ceil(dense_rows / BM)
  int out_f32;            // C is fp32 (act must be none); else C has the input dtype
  const int32_t* a_gather;  // routed problems: A row of compact row r is a_gather[r] (nullptr:
                            // row r itself); lets GEMM 1 read the tokens of x directly
  // K-major operands: stored [K][rows] with rows contiguous and lda / ldb the pitch between
  // consecutive k (elements).  Rows of k >= K read as zeros, so K need not be a multiple of
  // the GEMM's K chunk.  Not combined with a_gather, K segments or a gated B.
  int a_kmajor, b_kmajor;
  // Fused activation gradient (dgrad of GEMM 2): 0 = off, else 1 + the activation code.  The
  // product d (the gradient at the activation's output) is written as d * act'(z) to C, where
  // z has C's layout (same offsets and pitch); gated: z holds [g | u] with the u half
  // glu_h columns after the g half, and C receives dg there and du glu_h columns later.
  const void* z;
  int dact;
  // With the activation gradient, routed tiles only: row r of the product (compact row
  // row0 + r) is first multiplied by row_scale[row0 + r] (nullable), and the unscaled product
  // is dotted with hdot (pitch ldh, compact rows, nullable) over each n-tile into
  // dwp[(row0 + r) * dwp_ld + n-tile].
  const float* row_scale;
  const void* hdot;
  int64_t ldh;
  float* dwp;
  int dwp_ld;
  // Pre-activation output (training forward of GEMM 1 with a GELU or SwiGLU activation;
  // nullptr: none): the tile's accumulators before the activation, rounded to C's dtype, at
  // zout with pitch ldz and C's column offsets; gated problems write each output's gate
  // pre-activation at its gate row's column of the stacked [G; U] weight and its up
  // pre-activation glu_h columns later.
  void* zout;
  int64_t ldz;
};

struct GemmArgs {
  GemmProblem p0, p1;
  int nprob;              // 1 or 2 (p1 is always dense)
  int dtype;
  int group_m;            // m-tiles that sweep the n-tiles together (0: the kernel's default)
  int plain;              // one-problem launch order: 0 XCD ranges, 1 plain, 2 expert-synchronous
};

// Gather + gate-weighted sum + shared experts + residual, and (block 0) the final aux.
struct CombineArgs {
  const void* x;          // [N, M] T
  const void* o;          // [R, M] T expert outputs in compact order
  const void* o_sh;       // [N, M] T shared-expert sum or nullptr
  const int32_t* row;     // [N, k]
  const float* topk_w;    // [N, k]
  void* y;                // [N, M] T
  const double* Pg;       // [G][E]
  const int32_t* Cg;      // [G][E]
  float* aux;             // scalar
  const double* zpart;    // [nblocks] router-block partial sums of logsumexp^2
  float* z_loss;          // scalar or nullptr (not requested)
  float* dev_loss;        // scalar or nullptr (not requested)
  int nblocks;
  int n_eg;               // expert groups of the device-level loss
  int N, M, k, residual, dtype, G, E, S;
  int tpb;                // tokens per combine block (set by launch_combine)
};

struct EmptyArgs {         // N == 0: zero the small outputs (aux, z_loss, dev_loss nullable)
  int32_t* count; int32_t* offset; int32_t* stats; float* aux; float* z_loss; float* dev_loss;
  int G, E;
};

// ---- backward pass (moe_backward.hip)


struct BwdSetupArgs {      // batched GEMM entries of the backward (built on the device)
  const int32_t* offset;   // [E+1] expert offsets of the compact buffer
  BatchEntry* dw2; BatchEntry* dw1;  // [E + Es * nshared] weight gradients (routed, then the
                                     // shared experts' token ranges)
  BatchEntry* dhsh;                  // [Es] shared experts' dz
  BatchEntry* dwg;                   // [nsplit] token ranges of the router weight gradient
  int E, Es, M, H, H1, N, Ep, nsplit, ksplit, nshared, kshared;
};

struct RouterBwdArgs {
  const float* logits; const int32_t* topk_idx; const float* dw; const int32_t* Cg;
  float* dl;
  float coef_aux, coef_z, coef_dev, norm_p;
  int N, E, k, G, S, norm, n_eg;
};

struct DwgArgs {           // dbg = column sums of dl (two passes, fixed order)
  const float* dl; float* partb; float* dbg;
  int N, E, nchunks;
};

struct DxArgs {            // dx = [res] dy + sum_j dx_rows[row] + dx_shared + router term
  const void* dy; const void* dxr; const void* dxsh; const void* dxrt;
  const int32_t* row; void* dx;
  int N, M, k, residual, dtype;
};

struct RouterPrepArgs {    // dlp [N, Ep] = dl in the layer dtype, zero beyond E
  const float* dl; void* dlp;
  int N, E, Ep, dtype;
};

hipError_t launch_bwd_setup(const BwdSetupArgs& a, hipStream_t s);
hipError_t launch_router_bwd(const RouterBwdArgs& a, hipStream_t s);
hipError_t launch_dbg(const DwgArgs& a, hipStream_t s);
// out[i] = sum over s < S of part[s][i], in order of s (n a multiple of 4)
// dw[i] = sum over t < ntn of dwp[row[i] * ntn + t] in order of t (0 where row[i] < 0)
hipError_t launch_dw_reduce(const int32_t* row, const float* dwp, float* dw, int64_t n, int ntn,
                            hipStream_t s);
hipError_t launch_split_reduce(const float* part, float* out, int64_t n, int S, hipStream_t s);
hipError_t launch_router_dgrad_prep(const RouterPrepArgs& a, hipStream_t s);
hipError_t launch_dx_final(const DxArgs& a, hipStream_t s);
hipError_t launch_zero(float* p, int64_t n, hipStream_t s);

int gemm_block_m(int dtype);                           // BM of the expert GEMM tiles
int gemm_block_n(int dtype, int act);                  // output columns per tile
// m-tile group of a routed launch whose experts hold at most max_rows rows each: one expert's
// m-tiles when they are fewer than the default group, so that a group's concurrent tiles
// cover all n-tiles of one expert instead of a few n-tiles of several experts.
int gemm_group_m(int dtype, int64_t max_rows);

hipError_t launch_router(const RouterArgs& a, hipStream_t s);
hipError_t launch_gate_scan(const ScanArgs& a, hipStream_t s);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
hipError_t launch_expert_gemm(const GemmArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_aux_only(const CombineArgs& a, hipStream_t s);
hipError_t launch_empty(const EmptyArgs& a, hipStream_t s);

// moe_forward with a given workspace (moe_api.cpp), shared by the entry points;
// check_only: run the host checks only (nothing is enqueued).
int forward_workspace(const moe_cfg* cfg, const void* x, const void* Wg, const float* bg,
                      const void* W1, const void* W2, const float* u, void* y, float* aux,
                      const moe_meta* m, void* workspace, size_t wbytes, void* stream,
                      bool check_only);

}  // namespace moe
