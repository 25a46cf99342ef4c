// moe_expert_ffn: grouped (ragged) GEMM of the expert FFNs.
//
// [GShard] "MoE Transformer": every expert is a two-layer network of the dense FFN's shape,
// here act(x W1_e^T) W2_e^T.  The dispatched rows sit expert-major in one compact buffer,
// so each expert's rows form one contiguous GEMM; a tile list built on the device
// (offsets_kernel) cuts them into BM-row tiles, and one launch covers every expert, with
// no padding rows computed beyond the last partial tile of each expert and no host sync.
// A second, dense problem (the shared experts, fused into one FFN whose hidden layer is the
// concatenation of theirs, [11-868 #12] "機制：Transformer 各部分怎麼切") can ride in the
// same launch.
//
// bf16 kernel (gfx950): 256 x 256 tiles (the last n-tile of a problem may be partial), 8 waves, v_mfma_f32_32x32x16_bf16,
// operands loaded global -> LDS directly (buffer_load ... lds) through two stages of 64-deep
// K chunks, an LDS-staged epilogue with the activation fused, and an XCD-aware tile order:
// each XCD (blocks b with equal b % 8) receives a contiguous range of tiles, inside which 8
// m-tiles sweep the n-tiles together (L2 reuse of weight tiles across an expert's row tiles
// and of row tiles across n-tiles).  Details at gemm_bf16_kernel.
// fp32 kernel: a 64 x 64 x 16 FMA tile for the fp32 layers (the fp32 MFMA and fp32 vector
// peaks are equal on this chip).
//
// Gated experts ([Lec16] "DeepSeek V3 MoE (670B)": (Swish(x W1) * (x W2)) W3) run their two
// input projections as one GEMM over the stacked weight: a tile's B rows are arranged so
// that the lane (bf16) or thread (fp32) holding the gate pre-activation of an output also
// holds its up pre-activation, and the epilogue writes Swish(g) * u, half as many columns
// as the tile computed.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
// K depth of one LDS stage of the bf16 GEMM and the number of stages.  64 x 2 (one 128-byte
// line per operand row per chunk) measured fastest; 32 x 4 and 32 x 5 keep more chunks in
// flight but split every line over two requests and were 7-8% slower.
#ifndef MOE_GEMM_BK
#define MOE_GEMM_BK 64
#define MOE_GEMM_STAGES 2
#endif
constexpr int kGemmBK = MOE_GEMM_BK;
constexpr int kGemmStages = MOE_GEMM_STAGES;
// m-tiles that sweep the n-tiles together inside one XCD's range of tiles
#ifndef MOE_GEMM_GROUP_M
#define MOE_GEMM_GROUP_M 8
#endif
constexpr int kGemmGroupM = MOE_GEMM_GROUP_M;
// waves along N of the bf16 tile (2 x WN waves; 4: 128 x 64 per wave, 2: 128 x 128)
#ifndef MOE_GEMM_WN
#define MOE_GEMM_WN 4
#endif
constexpr int kGemmWN = MOE_GEMM_WN;
// two-stage K loop with fragments read one step ahead, interleaved with the MFMAs
#ifndef MOE_GEMM_PIPELINED
#define MOE_GEMM_PIPELINED 1
#endif
constexpr bool kGemmPipelined = MOE_GEMM_PIPELINED;
// pipelined loop: the wm = 1 waves refill the freed stage after the last step's MFMAs rather
// than before them
#ifndef MOE_GEMM_STAGGER
#define MOE_GEMM_STAGGER 1
#endif
constexpr bool kGemmStagger = MOE_GEMM_STAGGER;
// fp32 output tiles (weight gradients) staged per wave instead of per block
#ifndef MOE_GEMM_F32_WAVE_STAGING
#define MOE_GEMM_F32_WAVE_STAGING 1
#endif

struct Job {
  const char* A;   // first row of the tile (bytes)
  int64_t lda;     // bytes
  const char* B;   // first row of the n-tile of expert e (bytes)
  int64_t ldb;     // bytes
  int64_t kseg;    // elements
  int64_t segb;    // bytes between K segments of B
  char* C;         // first row, first column of the tile (bytes)
  int64_t ldc;     // bytes
  int K;
  int nrows;       // valid rows of the tile
  int ncols;       // valid columns of the tile (the last n-tile of a problem may be partial)
  int rows_left;   // rows readable from the tile's first row (clamp)
  int act;
  int64_t upb;     // gated problems: bytes from a gate row of B to its up row
  const int32_t* gather;  // A row of tile row r is gather[r] (A then points at row 0), or nullptr
  int64_t a_bytes;        // gathered A: readable bytes from A
  // K-major operands ([K][rows], lda / ldb = pitch between k): A / B point at the tile's first
  // row of k = 0
  int akm, bkm;
  const char* Z;   // fused activation gradient: z at the tile's first element (C's layout)
  int64_t zup;     // gated: bytes from a g column to its u column (in z and in C)
  const float* rs; // row scales from the tile's first row, or nullptr
  const char* Hd;  // h at the tile's first row and column (pitch ldhb), or nullptr
  int64_t ldhb;
  float* dwp;      // dot partials of the tile's first row and n-tile (row pitch dwp_ld)
  int dwp_ld;
  char* Zo;        // pre-activation output at the tile's first row and column (or its gate
                   // column), or nullptr; the up half of a gated tile is zup bytes later
  int64_t ldzb;    // bytes
};

// Load through the constant address space: for tables no kernel of this file writes (tile
// lists, batch entries, tile counts), so that a uniform address gives a scalar load even
// after the kernel has stored to global memory.
template <class T>
__device__ __forceinline__ T load_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}
__device__ __forceinline__ TileDesc load_const(const TileDesc* p) {
  const int32_t* q = reinterpret_cast<const int32_t*>(p);
  return TileDesc{load_const(q), load_const(q + 1), load_const(q + 2), 0};
}
__device__ __forceinline__ BatchEntry load_const(const BatchEntry* p) {
  const int64_t* q = reinterpret_cast<const int64_t*>(p);
  return BatchEntry{load_const(q), load_const(q + 1), load_const(q + 2),
                    load_const(reinterpret_cast<const int32_t*>(q + 3)), 0};
}

// BN = output columns per tile (a gated tile computes 2 BN columns of A . B^T).  The block ->
// tile order (XCD ranges, dealt batched entries, m-tile groups) is tile_coord's.
template <int BM, int BN, int ESZ>
__device__ __forceinline__ bool decode_tile(const GemmArgs& g, Job& j, int bid) {
  const int nt0 = (g.p0.N + BN - 1) / BN;
  const int mt0 = g.p0.tiles ? load_const(g.p0.num_tiles) : g.p0.max_tiles;
  const int nt1 = g.nprob > 1 ? (g.p1.N + BN - 1) / BN : 0;
  const int mt1 = g.nprob > 1 ? g.p1.max_tiles : 0;
  const bool batched = g.p0.batch && (g.nprob == 1 || g.p1.batch);
  const TileSpace sp = tile_space(mt0, nt0, mt1, nt1, g.nprob, batched,
                                  (g.p0.dense_rows + BM - 1) / BM,
                                  (g.p1.dense_rows + BM - 1) / BM, g.plain);
  TileCoord tc;
  if (!tile_coord(sp, bid, g.group_m > 0 ? g.group_m : kGemmGroupM, tc)) return false;
  const bool second = tc.prob == 1;
  const int mt = tc.mt, nt = tc.nt;

  const GemmProblem& P = second ? g.p1 : g.p0;
  int e = 0, row0, nrows, K = P.K;
  int64_t aoff = 0, boff = 0, coff = 0;  // batched entries: element offsets
  if (P.tiles) {
    const TileDesc d = load_const(P.tiles + mt);
    e = d.expert; row0 = d.row0; nrows = d.nrows;
  } else if (P.batch) {
    int be;
    batch_tile(mt, P.dense_rows, BM, be, row0, nrows);
    const BatchEntry d = load_const(P.batch + be);
    aoff = d.a_off; boff = d.b_off; coff = d.c_off; K = d.K;
  } else {
    row0 = mt * BM; nrows = min(BM, P.dense_rows - row0);
  }
  const int osz = P.out_f32 ? 4 : ESZ;
  j.lda = P.lda * ESZ;
  j.gather = P.a_gather ? P.a_gather + row0 : nullptr;
  j.a_bytes = static_cast<int64_t>(P.a_rows) * j.lda;
  j.akm = P.a_kmajor;
  j.bkm = P.b_kmajor;
  j.A = static_cast<const char*>(P.A) + aoff * ESZ +
        (P.a_kmajor ? static_cast<int64_t>(row0) * ESZ
                    : P.a_gather ? 0 : static_cast<int64_t>(row0) * j.lda);
  j.ldb = P.ldb * ESZ;
  const int c0 = nt * BN;
  // first B row of the tile: output column c0, or for gated problems its gate row
  const int64_t brow = P.act == kActSwiglu
      ? static_cast<int64_t>(c0 / P.glu_h) * 2 * P.glu_h + c0 % P.glu_h : c0;
  j.B = static_cast<const char*>(P.B) + (static_cast<int64_t>(e) * P.b_stride + boff) * ESZ +
        (P.b_kmajor ? static_cast<int64_t>(c0) * ESZ : brow * j.ldb);
  j.upb = static_cast<int64_t>(P.glu_h) * j.ldb;
  j.kseg = P.kseg;
  j.segb = P.seg_stride * ESZ;
  j.ldc = P.ldc * osz;
  j.C = static_cast<char*>(P.C) + coff * osz + static_cast<int64_t>(row0) * j.ldc +
        static_cast<int64_t>(c0) * osz;
  j.Z = P.z ? static_cast<const char*>(P.z) + (j.C - static_cast<char*>(P.C)) : nullptr;
  j.rs = P.row_scale ? P.row_scale + row0 : nullptr;
  j.ldhb = P.ldh * osz;
  j.Hd = P.hdot ? static_cast<const char*>(P.hdot) + static_cast<int64_t>(row0) * j.ldhb +
                      static_cast<int64_t>(c0) * osz
                : nullptr;
  j.dwp = P.dwp ? P.dwp + static_cast<int64_t>(row0) * P.dwp_ld + nt : nullptr;
  j.dwp_ld = P.dwp_ld;
  j.ldzb = P.ldz * osz;
  j.Zo = P.zout ? static_cast<char*>(P.zout) + static_cast<int64_t>(row0) * j.ldzb +
                      (P.act == kActSwiglu ? brow : c0) * osz
                : nullptr;
  j.zup = static_cast<int64_t>(P.glu_h) * osz;
  j.K = K;
  j.nrows = nrows;
  j.ncols = min(BN, P.N - nt * BN);
  j.rows_left = P.a_rows - row0;
  j.act = P.act;
  return true;
}

// Byte offset of K element kk inside a (possibly segmented) B row.
__device__ __forceinline__ int64_t bseg_offset(const Job& j, int kk, int esz) {
  const int64_t seg = kk / j.kseg;
  return seg * j.segb + (kk - seg * j.kseg) * esz;
}

// Workgroup barrier for LDS hand-offs only: wait for this wave's LDS operations, then
// s_barrier.  Unlike __syncthreads() it carries no global-memory fence, so global loads in
// flight are not drained by it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads past the end return 0 and stores past
// it are dropped by the hardware.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           0x00020000);
}

// XOR pattern of the 16-byte columns of LDS row r, for rows of ROW bytes.  The LDS serves
// a ds_read_b128 16 lanes at a time from 64 banks; the fragment reads take one column from
// 16 consecutive rows, which must then cover every bank once.
//  * 128-byte rows (8 columns): rows r and r + 2 share banks; ((r >> 1) & 7) ^ ((r & 1) << 2)
//    gives the 8 row pairs 8 distinct columns, the two rows of a pair differing in bit 2;
//  * 64-byte rows (4 columns): rows r and r + 4 share banks; (r >> 2) & 3 gives the 4 rows
//    of each bank class 4 distinct columns.
template <int ROW>
__device__ __forceinline__ int lds_swz(int r) {
  static_assert(ROW == 128 || ROW == 64, "LDS row size");
  if (ROW == 128) return ((r >> 1) & 7) ^ ((r & 1) << 2);
  return (r >> 2) & 3;
}

template <int ACT>
__device__ __forceinline__ float act_fn(float z) {
  if (ACT == kActRelu) return fmaxf(z, 0.0f);
  if (ACT == kActGelu) return gelu_erf(z);
  return z;
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding" (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left at their no-wait maxima).
#define MOE_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from a raw buffer straight into LDS (lane i -> lds + 16 i).  Kept out of
// lambdas: the host compilation pass drops the kernel's launch stub when this builtin is
// called from inside one.
__device__ __forceinline__ void dma16(rsrc_t r, unsigned char* lds, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// Expert GEMM tile: C[BM, BN] = act(A[BM, K] . B[BN, K]^T), bf16 in, fp32 accumulate, bf16 out.
//  * 2 x WN waves; wave (wm, wn) owns rows [wm BM/2, +BM/2) and columns [wn BN/WN, +BN/WN) as
//    v_mfma_f32_32x32x16_bf16 tiles (the weight fragment is the first operand, so a lane holds
//    one token row and runs of 4 features);
//  * K advances in chunks of BK through NST LDS stages of BK*2-byte rows.  Operands go from
//    global memory straight into LDS (buffer_load ... lds, 16 bytes per lane), NST - 1 chunks
//    in flight ahead of the one being multiplied (the loads take longer than one chunk of
//    MFMA work under full load).  Lane i of a load instruction writes LDS unit i, so the XOR
//    column swizzle is applied on the global side: LDS unit (row r, column p) receives
//    global column p ^ lds_swz(r);
//  * a barrier without a global-memory fence separates the stages, so the loads in flight are
//    never drained by it; each wave waits (vmcnt) only for its own part of the chunk it is
//    about to read;
//  * the epilogue applies the activation, packs bf16 and stages the tile in LDS (16-byte
//    columns XOR (row % columns)), then writes whole rows, 16 bytes per lane;
//  * gated (ACT == kActSwiglu): LDS B rows [64 s, 64 s + 32) hold the gate rows of output
//    columns [32 s, 32 s + 32) and rows [64 s + 32, 64 s + 64) their up rows, so wave wn's two
//    32-column MFMA blocks are the gate and up halves of the same 32 outputs, held by the
//    same lanes in the same registers; the tile writes BN / 2 columns.
template <int BM_, int BN_, int WN_, int BK_, int NST_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, WN = WN_, BK = BK_, NST = NST_;
  static constexpr int ROW = BK * 2, CPR = ROW / 16;  // bytes and 16-byte columns per LDS row
  static constexpr int NT = 128 * WN, NW = 2 * WN;
  static constexpr int STAGE = (BM + BN) * ROW;
  static constexpr int WTM = BM / 2, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int AQ = BM * ROW / 1024 / NW, BQ = BN * ROW / 1024 / NW;  // loads per wave/chunk
  static constexpr int Q = AQ + BQ;
  static_assert(NST >= 2 && NST <= 5 && BK * (NST - 1) <= 128, "K % 128 == 0 covers the prologue");
  static_assert(AQ * NW * 1024 == BM * ROW && BQ * NW * 1024 == BN * ROW, "tile/wave split");
};

// Where one tile's operand chunks come from: buffer resources, this lane's byte offsets for
// its load slots, and the K position of B inside its current segment.
template <class T>
struct Feed {
  rsrc_t ra, rb;
  uint32_t aoff[T::AQ], boff[T::BQ];
  int kin;          // elements into the current B segment
  uint32_t segoff;  // byte offset of that segment
  int kseg;         // elements per B segment
  uint32_t segb;    // bytes between B segments
  uint32_t kstepa, kstepb;  // K-major operands: bytes per K chunk
};

// K-major operand tiles in LDS: BK rows (one per k) of TILE * 2 bytes whose 16-byte units
// are XOR-permuted by kmaj_swz(k), so that the four consecutive k one transposed read covers
// fall on distinct banks.  The DMA applies the permutation on the global side.
__device__ __forceinline__ int kmaj_swz(int k) { return (k & 3) << 2; }

// Load slot q of wave w fills LDS units [(w + NW q) 64, +64) of its operand: for a row-major
// operand unit u is row u / CPR, physical column u % CPR; for a K-major one, k-row u / UPR.
template <class T, bool GLU, bool AKM, bool BKM>
__device__ __forceinline__ void feed_init(const Job& j, int w, int lane, Feed<T>& f) {
  const uint32_t lda = static_cast<uint32_t>(j.lda), ldb = static_cast<uint32_t>(j.ldb);
  static_assert(!(GLU && BKM), "a gated B is row-major");
  // K-major operands: rows of k >= K read as zeros.  The range ends at the last k-row's valid
  // columns rounded up to 16 bytes: a 16-byte load that crosses the end of a buffer range
  // reads as zeros as a whole.  (Pitches are multiples of 16 bytes, so the rounded bytes stay
  // inside that row.)
  if (AKM) {
    f.ra = make_rsrc(j.A, j.K > 0 ? static_cast<int64_t>(j.K - 1) * j.lda + ((j.nrows * 2 + 15) & ~15)
                                  : 0);
    constexpr int UPR = T::BM * 2 / 16;
#pragma unroll
    for (int q = 0; q < T::AQ; ++q) {
      const int u = (w + T::NW * q) * 64 + lane, kr = u / UPR, c = (u % UPR) ^ kmaj_swz(kr);
      f.aoff[q] = kr * lda + c * 16;
    }
  } else {
    f.ra = make_rsrc(j.A, j.gather ? j.a_bytes : static_cast<int64_t>(j.nrows) * j.lda);
#pragma unroll
    for (int q = 0; q < T::AQ; ++q) {
      const int u = (w + T::NW * q) * 64 + lane, r = u / T::CPR;
      const int c = (u % T::CPR) ^ lds_swz<T::ROW>(r);
      // gathered rows: tile rows past nrows read row gather[0] (their outputs are not stored)
      const uint32_t ar = j.gather ? static_cast<uint32_t>(j.gather[r < j.nrows ? r : 0]) : r;
      f.aoff[q] = ar * lda + c * 16;
    }
  }
  if (BKM) {
    f.rb = make_rsrc(j.B, j.K > 0 ? static_cast<int64_t>(j.K - 1) * j.ldb + ((j.ncols * 2 + 15) & ~15)
                                  : 0);
    constexpr int UPR = T::BN * 2 / 16;
#pragma unroll
    for (int q = 0; q < T::BQ; ++q) {
      const int u = (w + T::NW * q) * 64 + lane, kr = u / UPR, c = (u % UPR) ^ kmaj_swz(kr);
      f.boff[q] = kr * ldb + c * 16;
    }
  } else {
    const int nseg = max(1, (j.K + static_cast<int>(j.kseg) - 1) / static_cast<int>(j.kseg));
    // Weight rows past the problem's N (a partial last n-tile) read as zeros.
    f.rb = make_rsrc(j.B, (nseg - 1) * j.segb + (GLU ? j.upb : 0) +
                              static_cast<int64_t>(j.ncols) * j.ldb);
#pragma unroll
    for (int q = 0; q < T::BQ; ++q) {
      const int u = (w + T::NW * q) * 64 + lane, r = u / T::CPR;
      const int c = (u % T::CPR) ^ lds_swz<T::ROW>(r);
      if (GLU)   // LDS row r: output column 32 (r / 64) + r % 32, gate or up half by bit 5
        f.boff[q] = ((r >> 6) * 32 + (r & 31)) * ldb +
                    ((r >> 5) & 1) * static_cast<uint32_t>(j.upb) + c * 16;
      else
        f.boff[q] = r * ldb + c * 16;
    }
  }
  f.kin = 0;
  f.segoff = 0;
  f.kseg = static_cast<int>(j.kseg);
  f.segb = static_cast<uint32_t>(j.segb);
  f.kstepa = static_cast<uint32_t>(T::BK) * lda;
  f.kstepb = static_cast<uint32_t>(T::BK) * ldb;
}

// Issue this wave's loads of the A half of K chunk kt into LDS at As.  K-major operands move
// by whole k rows, through the per-lane offset so that the buffer bounds see the k rows.
template <class T, bool AKM>
__device__ __forceinline__ void feed_issue_a(const Feed<T>& f, unsigned char* As, int w, int kt) {
  const uint32_t ka = static_cast<uint32_t>(kt) * (AKM ? f.kstepa : T::ROW);
#pragma unroll
  for (int q = 0; q < T::AQ; ++q) {
    if (AKM) dma16(f.ra, As + (w + T::NW * q) * 1024, f.aoff[q] + ka, 0);
    else dma16(f.ra, As + (w + T::NW * q) * 1024, f.aoff[q], ka);
  }
}

// Issue this wave's loads of the B half of K chunk kt into LDS at Bs (B chunks are issued in
// K order: a row-major B follows its K segments).
template <class T, bool BKM>
__device__ __forceinline__ void feed_issue_b(Feed<T>& f, unsigned char* Bs, int w, int kt) {
  if (BKM) {
    const uint32_t kb = static_cast<uint32_t>(kt) * f.kstepb;
#pragma unroll
    for (int q = 0; q < T::BQ; ++q) dma16(f.rb, Bs + (w + T::NW * q) * 1024, f.boff[q] + kb, 0);
    return;
  }
  const uint32_t kb = f.segoff + static_cast<uint32_t>(f.kin) * 2;
#pragma unroll
  for (int q = 0; q < T::BQ; ++q) dma16(f.rb, Bs + (w + T::NW * q) * 1024, f.boff[q], kb);
  f.kin += T::BK;
  const bool wrap = f.kin == f.kseg;
  f.kin = wrap ? 0 : f.kin;
  f.segoff += wrap ? f.segb : 0u;
}

// Issue K chunk kt (A then B) into one whole-chunk stage.
template <class T, bool AKM, bool BKM>
__device__ __forceinline__ void feed_issue(Feed<T>& f, unsigned char* stage, int w, int kt) {
  feed_issue_a<T, AKM>(f, stage, w, kt);
  feed_issue_b<T, BKM>(f, stage + T::BM * T::ROW, w, kt);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_ptr;

// MFMA operand fragment from a K-major tile with rows of RK bytes: row ibase + lane % 32,
// k = 16 s + 8 (lane / 32) + 0..7, by two ds_read_b64_tr_b16.  Within each 16-lane group
// that instruction hands lane i element i % 4 of the 8-byte loads of lanes 4 r + i / 4,
// r = 0..3: lane i addresses k-row k0 + i / 4 at columns c0 + 4 (i % 4) .. + 3 and receives
// column c0 + i of the k-rows k0 .. k0 + 3.
template <int RK>
__device__ __forceinline__ bf16x8 frag_kmajor(const unsigned char* S, int s, int ibase, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const int col = ibase + 16 * (g & 1) + 4 * (i & 3);
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = 16 * s + 8 * (g >> 1) + 4 * h + (i >> 2);
    const unsigned char* p = S + k * RK + (((col >> 3) ^ kmaj_swz(k)) << 4) + (col & 7) * 2;
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16_ptr)(const_cast<unsigned char*>(p)));
    const u32x2 x2 = __builtin_bit_cast(u32x2, v);
    out[2 * h] = x2[0];
    out[2 * h + 1] = x2[1];
  }
  return __builtin_bit_cast(bf16x8, out);
}

// Multiply one K chunk (A rows at As, B rows at Bs in LDS) into the wave's accumulators.
// arow / brow: the wave's first A and B fragment rows for this lane; sw: the column swizzle
// of those rows (row-major operands).
template <class T, bool AKM, bool BKM>
__device__ __forceinline__ void mma_chunk(const unsigned char* As, const unsigned char* Bs,
                                          int arow, int brow, int lane, int sw,
                                          f32x16 (&acc)[T::TN][T::TM]) {
#pragma unroll
  for (int s = 0; s < T::BK / 16; ++s) {
    const int phys = (((2 * s) + (lane >> 5)) ^ sw) * 16;
    bf16x8 af[T::TM], bfr[T::TN];
#pragma unroll
    for (int im = 0; im < T::TM; ++im)
      af[im] = AKM ? frag_kmajor<T::BM * 2>(As, s, arow - (lane & 31) + 32 * im, lane)
                   : *reinterpret_cast<const bf16x8*>(As + (arow + 32 * im) * T::ROW + phys);
#pragma unroll
    for (int jn = 0; jn < T::TN; ++jn)
      bfr[jn] = BKM ? frag_kmajor<T::BN * 2>(Bs, s, brow - (lane & 31) + 32 * jn, lane)
                    : *reinterpret_cast<const bf16x8*>(Bs + (brow + 32 * jn) * T::ROW + phys);
#pragma unroll
    for (int jn = 0; jn < T::TN; ++jn)
#pragma unroll
      for (int im = 0; im < T::TM; ++im)
        acc[jn][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jn], af[im], acc[jn][im],
                                                              0, 0, 0);
  }
}

// The same multiply split into its two halves, for the pipelined K loop: the fragments of
// one 16-deep step (row-major: one ds_read_b128 each; K-major: two transposed reads each) ...
template <class T, bool AKM, bool BKM>
__device__ __forceinline__ void read_step(const unsigned char* As, const unsigned char* Bs, int s,
                                          int arow, int brow, int lane, int sw,
                                          bf16x8 (&af)[T::TM], bf16x8 (&bfr)[T::TN]) {
  const int phys = (((2 * s) + (lane >> 5)) ^ sw) * 16;
#pragma unroll
  for (int im = 0; im < T::TM; ++im)
    af[im] = AKM ? frag_kmajor<T::BM * 2>(As, s, arow - (lane & 31) + 32 * im, lane)
                 : *reinterpret_cast<const bf16x8*>(As + (arow + 32 * im) * T::ROW + phys);
#pragma unroll
  for (int jn = 0; jn < T::TN; ++jn)
    bfr[jn] = BKM ? frag_kmajor<T::BN * 2>(Bs, s, brow - (lane & 31) + 32 * jn, lane)
                  : *reinterpret_cast<const bf16x8*>(Bs + (brow + 32 * jn) * T::ROW + phys);
}
// ... and its MFMAs.
template <class T>
__device__ __forceinline__ void mfma_step(const bf16x8 (&af)[T::TM], const bf16x8 (&bfr)[T::TN],
                                          f32x16 (&acc)[T::TN][T::TM]) {
#pragma unroll
  for (int jn = 0; jn < T::TN; ++jn)
#pragma unroll
    for (int im = 0; im < T::TM; ++im)
      acc[jn][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jn], af[im], acc[jn][im], 0, 0, 0);
}
// Instruction order inside one step of the pipelined loop: the next step's LDS reads spread one
// after each MFMA (then the remaining MFMAs), so the reads run in the MFMA shadow instead of in
// a burst the MFMAs wait behind.
template <int NRD, int NMF>
__device__ __forceinline__ void interleave_step() {
#pragma unroll
  for (int i = 0; i < NRD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one DS read
    if (i < NMF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
  }
  if (NMF > NRD) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD, 0);
}

// 8 bf16 values (one 16-byte chunk) to fp32 and back.
__device__ __forceinline__ void unpack_bf16x8(u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    f[2 * x] = __builtin_bit_cast(float, v[x] << 16);
    f[2 * x + 1] = __builtin_bit_cast(float, v[x] & 0xffff0000u);
  }
}
__device__ __forceinline__ u32x4 pack_bf16x8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int x = 0; x < 4; ++x) v[x] = pack_bf16x2(f[2 * x], f[2 * x + 1]);
  return v;
}
// Activation gradient on 8 bf16 values d of the product scaled by s: returns s d act'(z)
// (gated: dg = s d u Swish'(g), with du = s d Swish(g) in du; z = g, u the up
// pre-activations, unused otherwise).
template <int DACT>
__device__ __forceinline__ u32x4 dact_vals(u32x4 d, u32x4 z, u32x4 u, float scale, u32x4& du) {
  float dv[8], zv[8], o[8];
  unpack_bf16x8(d, dv);
#pragma unroll
  for (int x = 0; x < 8; ++x) dv[x] *= scale;
  unpack_bf16x8(z, zv);
  if (DACT == kActSwiglu) {
    float uv[8], dd[8];
    unpack_bf16x8(u, uv);
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      o[x] = dv[x] * uv[x] * swish_grad(zv[x]);
      dd[x] = dv[x] * swish(zv[x]);
    }
    du = pack_bf16x8(dd);
  } else {
#pragma unroll
    for (int x = 0; x < 8; ++x)
      o[x] = DACT == kActGelu ? dv[x] * gelu_grad(zv[x]) : (zv[x] > 0.0f ? dv[x] : 0.0f);
  }
  return pack_bf16x8(o);
}

// bf16 epilogue through LDS: D[feature][token] -> tile[token][feature] (rows of OUTN*2 bytes,
// NCH 16-byte columns XOR (row % NCH)), then whole rows to global memory, 16 bytes per lane.
// The staging area holds STG bytes; a tile that does not fit goes through it in passes of
// whole wave-row blocks.  The caller has made the area free (a barrier after its last read);
// on return every wave's last reads of it are issued but not waited for.
// RAW = 1 stores the accumulators without the activation (gated tiles: the gate halves),
// RAW = 2 the up halves of a gated tile.
template <class T, int ACT, int STG, bool F32 = false, int DACT = -1, int RAW = 0>
__device__ __forceinline__ void store_tile(const Job& j, f32x16 (&acc)[T::TN][T::TM],
                                           unsigned char* stg, int t, int lane, int wm,
                                           int wn) {
  constexpr bool GLU = ACT == kActSwiglu;
  static_assert(!F32 || ACT == kActNone, "fp32 output carries no activation");
  constexpr int OUTN = GLU ? T::BN / 2 : T::BN;
  constexpr int RB = OUTN * (F32 ? 4 : 2), NCH = RB / 16;
  constexpr int TNO = GLU ? T::TN / 2 : T::TN, WTNO = OUTN / T::WN;
  constexpr int RP = STG / RB < T::BM ? STG / RB : T::BM;  // rows per pass
  static_assert((NCH & (NCH - 1)) == 0, "power-of-two column count");
  static_assert(RP % T::WTM == 0 && T::BM % RP == 0, "passes of whole wave-row blocks");
  static_assert(RAW == 0 || (!F32 && DACT < 0), "raw pre-activations: bf16 output only");
  static_assert(RAW < 2 || GLU, "up halves exist in gated tiles only");
  auto out = [&](int jo, int im, int x) {
    if (RAW == 1) return GLU ? acc[2 * jo][im][x] : acc[jo][im][x];
    if (RAW == 2) return acc[2 * jo + 1][im][x];
    if (GLU) return swish(acc[2 * jo][im][x]) * acc[2 * jo + 1][im][x];
    return act_fn<ACT>(acc[jo][im][x]);
  };
#if MOE_GEMM_F32_WAVE_STAGING
  if constexpr (F32 && DACT < 0 && RAW == 0) {
    // fp32 tiles (the weight gradients): each wave stages its own 128 x 32 blocks, one column
    // block jo at a time, in a private 16 KB region of the staging area and writes them back
    // as whole 128-byte row segments, so no block barrier holds any wave and all eight waves
    // stage at once.  Region rows are 128 bytes with their 16-byte columns XOR ((r >> 1) & 7):
    // the writes (16 rows x one column per 16 lanes) and the reads (2 rows x 8 columns) are
    // conflict-free.  A wave reads back only what it wrote, and its LDS operations complete
    // in order, so the stores' use of each read is the only wait.
    constexpr int RR = 128;   // bytes per region row: 32 fp32 columns
    static_assert(STG >= T::NW * T::WTM * RR, "a private staging region per wave");
    unsigned char* reg = stg + (t >> 6) * (T::WTM * RR);
#pragma unroll
    for (int jo = 0; jo < T::TN; ++jo) {
#pragma unroll
      for (int im = 0; im < T::TM; ++im) {
        const int r = 32 * im + (lane & 31);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int sg = 2 * qd + (lane >> 5);   // 16-byte column of the region row
          f32x4 v;
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] = acc[jo][im][4 * qd + x];
          *reinterpret_cast<f32x4*>(reg + r * RR + ((sg ^ ((r >> 1) & 7)) << 4)) = v;
        }
      }
      const int c0 = wn * (T::BN / T::WN) + 32 * jo;   // tile column of the block's column 0
#pragma unroll
      for (int q = 0; q < T::WTM / 8; ++q) {
        const int r = 8 * q + (lane >> 3), sg = lane & 7;
        const f32x4 v = *reinterpret_cast<const f32x4*>(reg + r * RR + ((sg ^ ((r >> 1) & 7)) << 4));
        const int row = wm * T::WTM + r, col = c0 + 4 * sg;
        if (row < j.nrows && col < j.ncols)
          __builtin_nontemporal_store(
              v, reinterpret_cast<f32x4*>(j.C + static_cast<int64_t>(row) * j.ldc + col * 4));
      }
    }
    return;
  }
#endif
  const int ncch = j.ncols / (F32 ? 4 : 8);   // valid 16-byte columns
  // Fused activation gradient, in batches of U row chunks per thread: every global load of a
  // batch (z, u for gated layers, h for the dot partials, the row scale) is issued before the
  // first of them is used, so a batch waits for one memory round trip, not U; the first
  // batch's loads are issued before the product is staged, so that round trip overlaps the
  // staging.  The loads are unconditional (chunks past the tile read its first chunk) and
  // masked where they are used: a load under a divergent branch, whose other side zeroes
  // the same registers, has to be waited for before the branch merges.  A half-wave covers
  // one staged row (NCH = 32 chunks), so the batch bounds are uniform over each half-wave
  // and its 32 lanes reduce the row's dot partial together.
  constexpr int U = DACT == kActSwiglu ? 4 : 8;   // gated: three loads per chunk
  u32x4 zv[U], uv[U], hv[U];
  float sc[U];
  const bool hz = j.Hd == j.Z && j.ldhb == j.ldc;   // ReLU: z is h
  auto dact_load = [&](int i0, int rows) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * T::NT;
      const int r = i / NCH, c = i - r * NCH;
      const bool ok = i < rows * NCH && c < ncch;
      const int64_t o = ok ? static_cast<int64_t>(r) * j.ldc + c * 16 : 0;
      zv[u] = *reinterpret_cast<const u32x4*>(j.Z + o);
      if (DACT == kActSwiglu) uv[u] = *reinterpret_cast<const u32x4*>(j.Z + o + j.zup);
      if (j.dwp && !hz)
        hv[u] = *reinterpret_cast<const u32x4*>(
            j.Hd + (ok ? static_cast<int64_t>(r) * j.ldhb + c * 16 : 0));
      sc[u] = j.rs ? j.rs[i < rows * NCH ? r : 0] : 1.0f;
    }
  };
  if constexpr (DACT >= 0) {
    static_assert(RP == T::BM && NCH == 32 && !F32, "one pass; one staged row per half-wave");
    dact_load(t, j.nrows);
  }
#pragma unroll
  for (int p = 0; p < T::BM / RP; ++p) {
    if (p > 0) lds_barrier();   // the previous pass has been read out
    if (wm * T::WTM / RP == p) {
#pragma unroll
      for (int im = 0; im < T::TM; ++im) {
        const int tok = wm * T::WTM + 32 * im + (lane & 31) - p * RP;
#pragma unroll
        for (int jo = 0; jo < TNO; ++jo) {
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int f = wn * WTNO + 32 * jo + 8 * qd + 4 * (lane >> 5);
            if (F32) {   // 4 fp32 features: one whole 16-byte column
              f32x4 v;
#pragma unroll
              for (int x = 0; x < 4; ++x) v[x] = acc[jo][im][4 * qd + x];
              const int ch = f >> 2;
              *reinterpret_cast<f32x4*>(stg + tok * RB + ((ch ^ (tok & (NCH - 1))) << 4)) = v;
            } else {
              u32x2 pk;
              pk[0] = pack_bf16x2(out(jo, im, 4 * qd + 0), out(jo, im, 4 * qd + 1));
              pk[1] = pack_bf16x2(out(jo, im, 4 * qd + 2), out(jo, im, 4 * qd + 3));
              const int ch = f >> 3, within = (f & 7) * 2;
              *reinterpret_cast<u32x2*>(stg + tok * RB + ((ch ^ (tok & (NCH - 1))) << 4) +
                                        within) = pk;
            }
          }
        }
      }
    }
    lds_barrier();
    const int rows = min(RP, j.nrows - p * RP);
    const int64_t poff = static_cast<int64_t>(p * RP) * j.ldc;
    char* C = j.C + poff;
    if constexpr (DACT >= 0) {
      for (int i0 = t;;) {
        u32x4 sv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {   // staged rows past the tile read row 0
          const int i = i0 + u * T::NT;
          const int r = i < rows * NCH ? i / NCH : 0, c = i % NCH;
          sv[u] = *reinterpret_cast<const u32x4*>(stg + r * RB + ((c ^ (r & (NCH - 1))) << 4));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * T::NT;
          if (i >= rows * NCH) break;
          const int r = i / NCH, c = i - r * NCH;
          if (j.dwp) {
            // <product row, h row> over this n-tile (zero past the valid columns)
            const u32x4 hvu = c < ncch ? (hz ? zv[u] : hv[u]) : u32x4{0u, 0u, 0u, 0u};
            float gv[8], hf[8], part = 0.f;
            unpack_bf16x8(sv[u], gv);
            unpack_bf16x8(hvu, hf);
#pragma unroll
            for (int x = 0; x < 8; ++x) part = fmaf(gv[x], hf[x], part);
            part = group_sum<16>(part);
            part += __shfl_xor(part, 16, 64);
            if (c == 0) j.dwp[static_cast<int64_t>(r) * j.dwp_ld] = part;
          }
          if (c >= ncch) continue;
          const int64_t o = static_cast<int64_t>(r) * j.ldc + c * 16;
          u32x4 du;
          const u32x4 dz = dact_vals<DACT>(sv[u], zv[u], uv[u], sc[u], du);
          *reinterpret_cast<u32x4*>(C + o) = dz;
          if (DACT == kActSwiglu) *reinterpret_cast<u32x4*>(C + o + j.zup) = du;
        }
        i0 += U * T::NT;
        if (i0 >= rows * NCH) break;
        dact_load(i0, rows);
      }
      continue;
    }
    // Whole staged rows out, 16 bytes per lane, in batches of 8 chunks per thread: the 8 LDS
    // reads (unconditional; chunks past the tile read row 0) are issued before the first
    // store, so a batch waits for one LDS round trip.
    constexpr int SB = 8;
    for (int i0 = t; i0 < rows * NCH; i0 += SB * T::NT) {
      u32x4 v[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int i = i0 + u * T::NT;
        const int r = i < rows * NCH ? i / NCH : 0, c = i % NCH;
        v[u] = *reinterpret_cast<const u32x4*>(stg + r * RB + ((c ^ (r & (NCH - 1))) << 4));
      }
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int i = i0 + u * T::NT;
        const int r = i / NCH, c = i - r * NCH;
        // streamed out (non-temporal): h and o are read back by the next kernel only, long
        // after L2 has turned over (0.7-2% off the whole layer)
        if (i < rows * NCH && c < ncch)
          __builtin_nontemporal_store(
              v[u], reinterpret_cast<u32x4*>(C + static_cast<int64_t>(r) * j.ldc + c * 16));
      }
    }
  }
}

// Workgroup barrier for LDS hand-offs, written with builtins so that the compiler's wait
// counters know every LDS and scalar-memory operation has completed at it: s_waitcnt
// lgkmcnt(0), then s_barrier (no global-memory fence, so loads in flight are not drained).
__device__ __forceinline__ void lds_barrier_visible() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt at their no-wait maxima
  __builtin_amdgcn_s_barrier();
}

// One K chunk of the pipelined two-stage loop (chunk kt in stage kt & 1).  Step s multiplies
// register set s & 1 while the reads of step s + 1 fill the other set.  At the last step, with
// NEXT (chunk kt + 1 exists), the block waits for chunk kt + 1, passes the barrier (every wave
// has read chunk kt's stage into registers), refills that stage with chunk kt + 2 (REFILL) and
// reads chunk kt + 1's first step, so no MFMA waits for a fragment read at a chunk boundary.
// The waves of tile half wm = 1 refill after their last MFMAs instead, so that each SIMD (one
// wave of each half) always has a wave issuing MFMAs while the other issues its loads.
// The last chunk (!NEXT) multiplies only its first ns 16-deep steps: with K-major operands K
// need not fill the chunk, and the steps past K would only add products of zeros.
template <class T, bool AKM, bool BKM, bool NEXT, bool REFILL>
__device__ __forceinline__ void k_chunk(Feed<T>& fd, unsigned char* smem, int kt, int w, int wm,
                                        int lane, int arow, int brow, int sw,
                                        bf16x8 (&fa)[2][T::TM], bf16x8 (&fb)[2][T::TN],
                                        f32x16 (&acc)[T::TN][T::TM], int ns = T::BK / 16) {
  constexpr int NS = T::BK / 16, SLOT = T::BM * T::ROW;
  constexpr int NRD = (T::TM + T::TN) * (AKM || BKM ? 2 : 1);   // wide upper bound
  constexpr int NMF = T::TM * T::TN;
  const int st = kt & 1;
  const unsigned char* S = smem + st * T::STAGE;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (!NEXT && s >= ns) break;   // uniform over the block
    if (s + 1 < NS) {
      if (NEXT || s + 1 < ns)
        read_step<T, AKM, BKM>(S, S + SLOT, s + 1, arow, brow, lane, sw, fa[(s + 1) & 1],
                               fb[(s + 1) & 1]);
    } else if (NEXT) {
      MOE_WAIT_VMCNT(0);
      lds_barrier_visible();
      if (REFILL && !(kGemmStagger && wm == 1))
        feed_issue<T, AKM, BKM>(fd, smem + st * T::STAGE, w, kt + 2);
      const unsigned char* Sn = smem + (st ^ 1) * T::STAGE;
      read_step<T, AKM, BKM>(Sn, Sn + SLOT, 0, arow, brow, lane, sw, fa[0], fb[0]);
    }
    mfma_step<T>(fa[s & 1], fb[s & 1], acc);
    interleave_step<NRD, NMF>();
    __builtin_amdgcn_sched_barrier(0);
    if (REFILL && kGemmStagger && s + 1 == NS && wm == 1) {
      feed_issue<T, AKM, BKM>(fd, smem + st * T::STAGE, w, kt + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One tile per block.
// KM: bit 0 = A is K-major, bit 1 = B is K-major.  DACT: fused activation gradient (-1: none).
// ZOUT: also store the pre-activations (training forward of GEMM 1).
template <int BM, int BN, int WN, int ACT, int BK, int NST, bool OUTF32, int KM, int DACT,
          bool ZOUT = false>
__global__ __launch_bounds__(128 * WN, 1) void gemm_bf16_kernel(GemmArgs g) {
  using T = TileShape<BM, BN, WN, BK, NST>;
  constexpr bool AKM = KM & 1, BKM = (KM >> 1) & 1;
  constexpr int SLOT = BM * T::ROW;   // one operand's rows of one chunk
  constexpr int SMEM = NST * T::STAGE > BM * BN * 2 ? NST * T::STAGE : BM * BN * 2;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];

  constexpr bool GLU = ACT == kActSwiglu;
  constexpr int OUTN = GLU ? BN / 2 : BN;    // output columns of the tile
  static_assert(!GLU || (BN / WN) % 64 == 0, "gated tiles: every wave holds gate/up block pairs");
  Job j;
  if (!decode_tile<BM, OUTN, 2>(g, j, blockIdx.x)) return;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  // Waves w and w + 4 share a SIMD: the second half's column blocks are rotated by WN / 2, so
  // that a tile whose valid columns end half-way still has one multiplying wave per SIMD.
  const int wm = w / WN, wn = (w % WN) ^ ((wm & 1) * (WN / 2));
  // A wave whose rows or columns all lie past the tile's valid block multiplies nothing.
  const bool live = wm * T::WTM < j.nrows && wn * (OUTN / WN) < j.ncols;
  Feed<T> fd;
  feed_init<T, GLU, AKM, BKM>(j, w, lane, fd);

  f32x16 acc[T::TN][T::TM];
#pragma unroll
  for (int jn = 0; jn < T::TN; ++jn)
#pragma unroll
    for (int im = 0; im < T::TM; ++im) acc[jn][im] = f32x16{};

  const int arow = wm * T::WTM + (lane & 31);
  const int brow = wn * T::WTN + (lane & 31);
  const int sw = lds_swz<T::ROW>(lane & 31);  // fragment rows are congruent to lane & 31 mod 16

  // Chunk kt lives in stage kt % NST.  Before multiplying chunk kt a wave lets the chunks
  // issued after it stay in flight (Q vector-memory operations each), then the barrier
  // makes every wave's part visible and frees the stage that chunk kt + NST - 1 refills.
  auto wait_chunk = [&](int ahead) {
    if (NST > 4 && ahead >= 3) MOE_WAIT_VMCNT(3 * T::Q);
    else if (NST > 3 && ahead >= 2) MOE_WAIT_VMCNT(2 * T::Q);
    else if (NST > 2 && ahead >= 1) MOE_WAIT_VMCNT(T::Q);
    else MOE_WAIT_VMCNT(0);
  };
  // 0 (a zero block) or >= NST - 1; a K-major operand's last chunk may be partial
  const int KT = (AKM || BKM) ? (j.K + BK - 1) / BK : j.K / BK;
  if (kGemmPipelined && NST == 2 && KT > 0) {
    // Two stages, fragments one 16-deep step ahead in two register sets.  Step s of chunk kt
    // multiplies set s & 1 while the reads of step s + 1 fill the other set; at the last
    // step the block waits for chunk kt + 1, passes the barrier (every wave has read chunk
    // kt's stage into registers by then), refills that stage with chunk kt + 2 and reads
    // chunk kt + 1's first step, so no MFMA waits for a fragment read at a chunk boundary.
    static_assert((BK / 16) % 2 == 0,
                  "an even number of steps per chunk keeps the register sets aligned");
    bf16x8 fa[2][T::TM], fb[2][T::TN];
    feed_issue<T, AKM, BKM>(fd, smem, w, 0);
    MOE_WAIT_VMCNT(0);
    lds_barrier_visible();
    if (KT > 1) feed_issue<T, AKM, BKM>(fd, smem + T::STAGE, w, 1);
    if (live) {
      read_step<T, AKM, BKM>(smem, smem + SLOT, 0, arow, brow, lane, sw, fa[0], fb[0]);
      // The steady state (chunks with a next chunk and one to refill) runs without a branch
      // around its LDS reads, so the compiler's waits count exactly the reads in flight; the
      // last two chunks are peeled.
      int kt = 0;
      for (; kt + 2 < KT; ++kt)
        k_chunk<T, AKM, BKM, true, true>(fd, smem, kt, w, wm, lane, arow, brow, sw, fa, fb, acc);
      if (kt + 1 < KT) {
        k_chunk<T, AKM, BKM, true, false>(fd, smem, kt, w, wm, lane, arow, brow, sw, fa, fb,
                                          acc);
        ++kt;
      }
      // steps of the last chunk that hold k < K (all of them unless an operand is K-major)
      const int ns = (AKM || BKM) ? min(BK / 16, (j.K - kt * BK + 15) / 16) : BK / 16;
      k_chunk<T, AKM, BKM, false, false>(fd, smem, kt, w, wm, lane, arow, brow, sw, fa, fb, acc,
                                         ns);
    } else {
      // the same loads and barriers as k_chunk, in the same order, without the MFMAs
      for (int kt = 0; kt + 1 < KT; ++kt) {
        MOE_WAIT_VMCNT(0);
        lds_barrier_visible();
        if (kt + 2 < KT) feed_issue<T, AKM, BKM>(fd, smem + (kt & 1) * T::STAGE, w, kt + 2);
      }
    }
  } else if (KT > 0) {
#pragma unroll
    for (int p = 0; p < NST - 1; ++p) feed_issue<T, AKM, BKM>(fd, smem + p * T::STAGE, w, p);
    int st = 0;
    for (int kt = 0; kt + NST - 1 < KT; ++kt) {
      wait_chunk(NST - 2);
      lds_barrier();
      const int sf = st == 0 ? NST - 1 : st - 1;  // (kt + NST - 1) % NST
      feed_issue<T, AKM, BKM>(fd, smem + sf * T::STAGE, w, kt + NST - 1);
      if (live)
        mma_chunk<T, AKM, BKM>(smem + st * T::STAGE, smem + st * T::STAGE + SLOT, arow, brow,
                               lane, sw, acc);
      st = st == NST - 1 ? 0 : st + 1;
    }
#pragma unroll
    for (int i = 0; i < NST - 1; ++i) {  // the last NST - 1 chunks: nothing left to issue
      wait_chunk(NST - 2 - i);
      lds_barrier();
      if (live)
        mma_chunk<T, AKM, BKM>(smem + st * T::STAGE, smem + st * T::STAGE + SLOT, arow, brow,
                               lane, sw, acc);
      st = st == NST - 1 ? 0 : st + 1;
    }
  }

  lds_barrier();
  // fp32 output (the weight-gradient GEMMs): rows of 1 KB, staged in passes of 128 rows
  store_tile<T, ACT, SMEM, OUTF32, DACT>(j, acc, smem, t, lane, wm, wn);
  if constexpr (ZOUT) {
    static_assert(!OUTF32 && DACT < 0 && ACT != kActNone, "pre-activations of GEMM 1");
    // the same staging, once more for the pre-activations (twice for gated tiles: gate
    // halves, then up halves)
    Job jz = j;
    jz.C = j.Zo;
    jz.ldc = j.ldzb;
    lds_barrier();
    store_tile<T, ACT, SMEM, false, -1, 1>(jz, acc, smem, t, lane, wm, wn);
    if constexpr (GLU) {
      jz.C = j.Zo + j.zup;
      lds_barrier();
      store_tile<T, ACT, SMEM, false, -1, 2>(jz, acc, smem, t, lane, wm, wn);
    }
  }
}

// Thread (ty, tx) accumulates rows 4 ty + i and LDS B columns 4 tx + jj.  Gated problems:
// LDS B column n holds output 2 (n / 4) + n % 2, its gate row for n % 4 < 2 and its up row
// otherwise, so a thread writes Swish(acc[i][jj]) * acc[i][jj + 2] for outputs 2 tx + jj,
// jj < 2 (32 output columns per tile).
template <bool GLU, int KM, int DACT>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs g) {
  constexpr int BM = 64, BN = 64, BK = 16, LDSW = 68;
  constexpr bool AKM = KM & 1, BKM = (KM >> 1) & 1;
  static_assert(!(GLU && BKM), "a gated B is row-major");
  __shared__ __attribute__((aligned(16))) float As[BK][LDSW];
  __shared__ __attribute__((aligned(16))) float Bs[BK][LDSW];
  Job j;
  if (!decode_tile<BM, GLU ? BN / 2 : BN, 4>(g, j, blockIdx.x)) return;
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  const int lr = t >> 2, lc = (t & 3) * 4;
  const int ar0 = lr < j.rows_left ? lr : j.rows_left - 1;
  const int ar = j.gather ? j.gather[lr < j.nrows ? lr : 0] : ar0;
  const char* ap = j.A + static_cast<int64_t>(ar) * j.lda + lc * 4;
  const int64_t boffs = GLU ? (2 * (lr >> 2) + (lr & 1)) * j.ldb + ((lr >> 1) & 1) * j.upb
                            : static_cast<int64_t>(lr) * j.ldb;
  const char* bp = j.B + boffs + lc * 4;
  // K-major operands: thread t loads k-row kt BK + t / 16, columns 4 (t % 16) .. + 3; k-rows
  // past K and columns past the tile's valid rows / columns load zeros
  const int kr = t >> 4, kc = (t & 15) * 4;
  float acc[4][4] = {};
  const int KT = (AKM || BKM) ? (j.K + BK - 1) / BK : j.K / BK;
  for (int kt = 0; kt < KT; ++kt) {
    const int kg = kt * BK + kr;
    if (AKM) {
      f32x4 av = {0.f, 0.f, 0.f, 0.f};
      if (kg < j.K && kc < j.nrows)
        av = *reinterpret_cast<const f32x4*>(j.A + static_cast<int64_t>(kg) * j.lda + kc * 4);
      *reinterpret_cast<f32x4*>(&As[kr][kc]) = av;
    } else {
      const f32x4 av = *reinterpret_cast<const f32x4*>(ap + static_cast<int64_t>(kt) * BK * 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) As[lc + q][lr] = av[q];
    }
    if (BKM) {
      f32x4 bv = {0.f, 0.f, 0.f, 0.f};
      if (kg < j.K && kc < j.ncols)
        bv = *reinterpret_cast<const f32x4*>(j.B + static_cast<int64_t>(kg) * j.ldb + kc * 4);
      *reinterpret_cast<f32x4*>(&Bs[kr][kc]) = bv;
    } else {
      const f32x4 bv = *reinterpret_cast<const f32x4*>(bp + bseg_offset(j, kt * BK, 4));
#pragma unroll
      for (int q = 0; q < 4; ++q) Bs[lc + q][lr] = bv[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&As[kk][ty * 4]);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(&Bs[kk][tx * 4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(a4[i], b4[jj], acc[i][jj]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= j.nrows) continue;
    if (GLU) {
      f32x2 o;
      o[0] = swish(acc[i][0]) * acc[i][2];
      o[1] = swish(acc[i][1]) * acc[i][3];
      *reinterpret_cast<f32x2*>(j.C + static_cast<int64_t>(r) * j.ldc + tx * 8) = o;
      if (j.Zo) {   // pre-activations: gate columns, and the up columns zup bytes later
        char* zr = j.Zo + static_cast<int64_t>(r) * j.ldzb + tx * 8;
        *reinterpret_cast<f32x2*>(zr) = f32x2{acc[i][0], acc[i][1]};
        *reinterpret_cast<f32x2*>(zr + j.zup) = f32x2{acc[i][2], acc[i][3]};
      }
    } else if (DACT >= 0) {   // fused activation gradient: z has C's layout
      const int64_t o = static_cast<int64_t>(r) * j.ldc + tx * 16;
      if (j.dwp) {   // <product row, h row> over this n-tile: the 16 lanes of row r
        const f32x4 hv = *reinterpret_cast<const f32x4*>(j.Hd + static_cast<int64_t>(r) * j.ldhb +
                                                         tx * 16);
        float part = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) part = fmaf(acc[i][jj], hv[jj], part);
        part = group_sum<16>(part);
        if (tx == 0) j.dwp[static_cast<int64_t>(r) * j.dwp_ld] = part;
      }
      const float sc = j.rs ? j.rs[r] : 1.0f;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[i][jj] *= sc;
      const f32x4 z = *reinterpret_cast<const f32x4*>(j.Z + o);
      f32x4 d;
      if (DACT == kActSwiglu) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(j.Z + o + j.zup);
        f32x4 du;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          d[jj] = acc[i][jj] * u[jj] * swish_grad(z[jj]);
          du[jj] = acc[i][jj] * swish(z[jj]);
        }
        *reinterpret_cast<f32x4*>(j.C + o + j.zup) = du;
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          d[jj] = DACT == kActGelu ? acc[i][jj] * gelu_grad(z[jj])
                                   : (z[jj] > 0.0f ? acc[i][jj] : 0.0f);
      }
      *reinterpret_cast<f32x4*>(j.C + o) = d;
    } else {
      f32x4 o;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) o[jj] = apply_act(acc[i][jj], j.act);
      *reinterpret_cast<f32x4*>(j.C + static_cast<int64_t>(r) * j.ldc + tx * 16) = o;
      if (j.Zo)
        *reinterpret_cast<f32x4*>(j.Zo + static_cast<int64_t>(r) * j.ldzb + tx * 16) =
            f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    }
  }
}

int grid_of(const GemmArgs& a, int BN) {
  int64_t total = static_cast<int64_t>(a.p0.max_tiles) * ((a.p0.N + BN - 1) / BN);
  if (a.nprob > 1) total += static_cast<int64_t>(a.p1.max_tiles) * ((a.p1.N + BN - 1) / BN);
  return static_cast<int>(total);
}

}  // namespace

int gemm_block_m(int dtype) { return dtype == 1 ? 256 : 64; }

int gemm_group_m(int dtype, int64_t max_rows) {
  const int64_t bm = gemm_block_m(dtype);
  const int64_t mt = (max_rows + bm - 1) / bm;
  return static_cast<int>(mt < 1 ? 1 : (mt < kGemmGroupM ? mt : kGemmGroupM));
}

// bf16: partial last n-tiles are masked; gated tiles write half the columns they compute.
int gemm_block_n(int dtype, int act) {
  const int bn = dtype == 1 ? 256 : 64;
  return act == kActSwiglu ? bn / 2 : bn;
}

hipError_t launch_expert_gemm(const GemmArgs& a, hipStream_t s) {
  const int act = a.p0.act;  // both problems of one launch share the activation and layouts
  const int km = (a.p0.a_kmajor ? 1 : 0) | (a.p0.b_kmajor ? 2 : 0);
  const int dact = a.p0.dact;  // 0: none, else 1 + activation code
  if (a.nprob > 1 && (((a.p1.a_kmajor ? 1 : 0) | (a.p1.b_kmajor ? 2 : 0)) != km ||
                      a.p1.dact != dact))
    return hipErrorInvalidValue;
  // supported layouts: row-major (any activation); K-major B (no activation, optionally the
  // fused activation gradient); K-major A and B (fp32 output)
  if ((km == 2 && act != kActNone) || km == 1 || (km == 3 && !a.p0.out_f32) ||
      ((km & 1) && a.p0.a_gather) || (dact && (km != 2 || !a.p0.z)) || dact < 0 || dact > 3 ||
      (a.p0.dwp && (!dact || !a.p0.hdot || !a.p0.tiles)))
    return hipErrorInvalidValue;
  // pre-activation output: GEMM 1 (row-major operands, bf16 or fp32 output of the input
  // dtype) with a GELU or SwiGLU activation, on both problems of the launch or neither
  const bool zout = a.p0.zout != nullptr;
  if ((a.nprob > 1 && (a.p1.zout != nullptr) != zout) ||
      (zout && (km != 0 || a.p0.out_f32 || dact || (act != kActGelu && act != kActSwiglu))))
    return hipErrorInvalidValue;
  const int grid = grid_of(a, gemm_block_n(a.dtype, act));
  if (grid == 0) return hipSuccess;
  const dim3 blk(128 * kGemmWN);
  if (a.dtype == 1) {
#define MOE_GEMM_LAUNCH(ACTV, OUTF, KMV, DACTV)                                             \
  hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, kGemmWN, ACTV, kGemmBK, kGemmStages, OUTF, \
                                       KMV, DACTV>),                                      \
                     dim3(grid), blk, 0, s, a)
#define MOE_GEMM_LAUNCH_Z(ACTV)                                                            \
  hipLaunchKernelGGL((gemm_bf16_kernel<256, 256, kGemmWN, ACTV, kGemmBK, kGemmStages, false, \
                                       0, -1, true>),                                     \
                     dim3(grid), blk, 0, s, a)
    if (zout) {
      if (act == kActGelu) MOE_GEMM_LAUNCH_Z(kActGelu);
      else MOE_GEMM_LAUNCH_Z(kActSwiglu);
    } else if (a.p0.out_f32) {
      if (km == 3) MOE_GEMM_LAUNCH(kActNone, true, 3, -1);
      else MOE_GEMM_LAUNCH(kActNone, true, 0, -1);
    } else if (km == 2) {
      if (dact == 1 + kActRelu) MOE_GEMM_LAUNCH(kActNone, false, 2, kActRelu);
      else if (dact == 1 + kActGelu) MOE_GEMM_LAUNCH(kActNone, false, 2, kActGelu);
      else if (dact == 1 + kActSwiglu) MOE_GEMM_LAUNCH(kActNone, false, 2, kActSwiglu);
      else MOE_GEMM_LAUNCH(kActNone, false, 2, -1);
    } else if (act == kActRelu) {
      MOE_GEMM_LAUNCH(kActRelu, false, 0, -1);
    } else if (act == kActGelu) {
      MOE_GEMM_LAUNCH(kActGelu, false, 0, -1);
    } else if (act == kActSwiglu) {
      MOE_GEMM_LAUNCH(kActSwiglu, false, 0, -1);
    } else {
      MOE_GEMM_LAUNCH(kActNone, false, 0, -1);
    }
#undef MOE_GEMM_LAUNCH
#undef MOE_GEMM_LAUNCH_Z
  } else if (act == kActSwiglu) {
    hipLaunchKernelGGL((gemm_f32_kernel<true, 0, -1>), dim3(grid), dim3(kThreads), 0, s, a);
  } else if (km == 3) {
    hipLaunchKernelGGL((gemm_f32_kernel<false, 3, -1>), dim3(grid), dim3(kThreads), 0, s, a);
  } else if (km == 2) {
#define MOE_F32_DACT(DACTV) \
  hipLaunchKernelGGL((gemm_f32_kernel<false, 2, DACTV>), dim3(grid), dim3(kThreads), 0, s, a)
    if (dact == 1 + kActRelu) MOE_F32_DACT(kActRelu);
    else if (dact == 1 + kActGelu) MOE_F32_DACT(kActGelu);
    else if (dact == 1 + kActSwiglu) MOE_F32_DACT(kActSwiglu);
    else MOE_F32_DACT(-1);
#undef MOE_F32_DACT
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<false, 0, -1>), dim3(grid), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
