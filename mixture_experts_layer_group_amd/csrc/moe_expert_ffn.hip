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
// bf16 kernel (gfx950):
//   * block tile BM x BN x 64, 256 threads = 2 x 2 waves, each wave (BM/2) x (BN/2) built
//     from v_mfma_f32_32x32x16_bf16 tiles with fp32 accumulators;
//   * A (token rows) and B (weight rows: W1 is [H, M], W2 is [M, H], so both operands are
//     K-contiguous) staged through LDS in two buffers of 128-byte rows whose 16-byte
//     columns are XOR-swizzled by (row & 7), so the fragment reads of 8 consecutive rows hit
//     distinct banks; the next K chunk is fetched into registers while the current one is
//     multiplied;
//   * the weight fragment is the MFMA's first operand, so every lane ends up owning one
//     token row and runs of 4 consecutive output features: the epilogue applies the
//     activation, rounds to bf16 and writes 8 bytes per run, masking rows past the tile;
//   * tiles are numbered so that each XCD (blocks b with equal b % 8) receives a contiguous
//     range, and inside a range 8 m-tiles sweep the n-tiles together (L2 reuse of the
//     weight tile across an expert's row tiles).
// fp32 kernel: a 64 x 64 x 16 FMA tile for the fp32 layers (the fp32 MFMA and fp32 vector
// peaks are equal on this chip).
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

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
  int rows_left;   // rows readable from the tile's first row (clamp)
  int act;
};

template <int BM, int BN, int ESZ>
__device__ __forceinline__ bool decode_tile(const GemmArgs& g, Job& j) {
  const int nt0 = g.p0.N / BN;
  const int mt0 = g.p0.tiles ? *g.p0.num_tiles : g.p0.max_tiles;
  const int tot0 = mt0 * nt0;
  const int nt1 = g.nprob > 1 ? g.p1.N / BN : 0;
  const int mt1 = g.nprob > 1 ? g.p1.max_tiles : 0;
  const int total = tot0 + mt1 * nt1;
  const int bid = blockIdx.x;
  if (bid >= total) return false;
  // Blocks are dispatched round-robin over the 8 XCDs (block b -> XCD b % 8); give every
  // XCD a contiguous range of tiles so neighbouring tiles share its L2.
  const int xcd = bid & 7, loc = bid >> 3, q = total >> 3, r = total & 7;
  const int pid = xcd * q + min(xcd, r) + loc;
  const bool second = pid >= tot0;
  const int lp = second ? pid - tot0 : pid;
  const int mts = second ? mt1 : mt0;
  const int nts = second ? nt1 : nt0;
  constexpr int GM = 8;
  const int per_group = GM * nts;
  const int grp = lp / per_group;
  const int first = grp * GM;
  const int gsz = min(mts - first, GM);
  const int in = lp - grp * per_group;
  const int mt = first + in % gsz;
  const int nt = in / gsz;

  const GemmProblem& P = second ? g.p1 : g.p0;
  int e, row0, nrows;
  if (P.tiles) {
    const TileDesc d = P.tiles[mt];
    e = d.expert; row0 = d.row0; nrows = d.nrows;
  } else {
    e = 0; row0 = mt * BM; nrows = min(BM, P.dense_rows - row0);
  }
  j.lda = P.lda * ESZ;
  j.A = static_cast<const char*>(P.A) + static_cast<int64_t>(row0) * j.lda;
  j.ldb = P.ldb * ESZ;
  j.B = static_cast<const char*>(P.B) + (static_cast<int64_t>(e) * P.b_stride) * ESZ +
        static_cast<int64_t>(nt) * BN * j.ldb;
  j.kseg = P.kseg;
  j.segb = P.seg_stride * ESZ;
  j.ldc = P.ldc * ESZ;
  j.C = static_cast<char*>(P.C) + static_cast<int64_t>(row0) * j.ldc +
        static_cast<int64_t>(nt) * BN * ESZ;
  j.K = P.K;
  j.nrows = nrows;
  j.rows_left = P.a_rows - row0;
  j.act = P.act;
  return true;
}

// Byte offset of K element kk inside a (possibly segmented) B row.
__device__ __forceinline__ int64_t bseg_offset(const Job& j, int kk, int esz) {
  const int64_t seg = kk / j.kseg;
  return seg * j.segb + (kk - seg * j.kseg) * esz;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads past the end return 0 and stores past
// it are dropped by the hardware.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 bload(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// XOR pattern of the 16-byte columns of LDS row r (128-byte rows).  Among any 8 aligned
// consecutive rows it takes 8 distinct values, and among any 16 aligned consecutive rows the
// rows of equal parity take 8 distinct values, so a ds_read_b128 of one column from 16
// consecutive rows touches every bank once whether the LDS serves 8 lanes per cycle from
// 32 banks or 16 lanes from 64 banks.
__device__ __forceinline__ int lds_swz(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

template <int ACT>
__device__ __forceinline__ float act_fn(float z) {
  if (ACT == 0) return fmaxf(z, 0.0f);
  if (ACT == 1) return gelu_erf(z);
  return z;
}

// Instruction order of one K chunk (a scheduling region between two barriers), given to
// the compiler as groups: the first k-step's fragment reads, then for every MFMA one other
// memory operation -- the next k-step's fragment reads first, global loads of the chunk
// after next during k-steps 0-1, LDS writes of the next chunk (whose loads are the oldest
// in flight) during k-steps 2-3.  MF = MFMAs per k-step, DR = fragment reads per k-step,
// NL = global loads, NW = LDS writes.
template <int MF, int DR, int NL, int NW>
__device__ __forceinline__ void sched_chunk() {
#pragma unroll
  for (int i = 0; i < DR; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  int loads = NL, writes = NW;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int m = 0; m < MF; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (s < 3 && m < DR) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      } else if (s < 2 && loads > 0) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        --loads;
      } else if (s >= 2 && writes > 0) {
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        --writes;
      }
    }
  }
}

template <int BM, int BN, int ACT>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WTM = BM / 2, WTN = BN / 2;   // wave tile (2 x 2 waves)
  constexpr int TM = WTM / 32, TN = WTN / 32; // 32x32 MFMA tiles per wave
  constexpr int ACH = BM / 32, BCH = BN / 32; // 16-byte chunks per thread per K chunk
  constexpr int ROW = 128;                    // bytes of one LDS row (64 bf16 of K)
  constexpr int STAGE = (BM + BN) * ROW;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

  Job j;
  if (!decode_tile<BM, BN, 2>(g, j)) return;

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int c = t & 7;                          // 16-byte column this thread loads
  const int rsub = t >> 3;                      // row within each 32-row slab
  const int scol = (c ^ lds_swz(rsub)) * 16;    // swizzled LDS column (rows r = rsub + 32 i)

  // A: only the tile's valid rows are addressable; the rest of the BM rows load as zeros.
  const uint32_t lda = static_cast<uint32_t>(j.lda), ldb = static_cast<uint32_t>(j.ldb);
  const rsrc_t ra_rs = make_rsrc(j.A, static_cast<int64_t>(j.nrows) * j.lda);
  const int nseg = (j.K + static_cast<int>(j.kseg) - 1) / static_cast<int>(j.kseg);
  const rsrc_t rb_rs = make_rsrc(j.B, (nseg - 1) * j.segb + static_cast<int64_t>(BN) * j.ldb);
  const uint32_t avoff = rsub * lda + c * 16;
  const uint32_t bvoff = rsub * ldb + c * 16;

  f32x16 acc[TN][TM];
#pragma unroll
  for (int jn = 0; jn < TN; ++jn)
#pragma unroll
    for (int im = 0; im < TM; ++im) acc[jn][im] = f32x16{};

  // Two register sets of prefetched K chunks: while chunk kt is multiplied out of LDS,
  // chunk kt+1 sits in one set (loaded one iteration earlier) and chunk kt+2 is in flight
  // into the other, so a global load has two chunks of MFMA work to arrive.
  u32x4 pa0[ACH], pb0[BCH], pa1[ACH], pb1[BCH];
  auto gload = [&](u32x4 (&pa)[ACH], u32x4 (&pb)[BCH], uint32_t ka, uint32_t kb) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) pa[i] = bload(ra_rs, avoff, ka + i * 32 * lda);
#pragma unroll
    for (int i = 0; i < BCH; ++i) pb[i] = bload(rb_rs, bvoff, kb + i * 32 * ldb);
  };
  auto sstore = [&](const u32x4 (&pa)[ACH], const u32x4 (&pb)[BCH], int st) {
    unsigned char* As = smem + st * STAGE;
    unsigned char* Bs = As + BM * ROW;
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      *reinterpret_cast<u32x4*>(As + (rsub + 32 * i) * ROW + scol) = pa[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i)
      *reinterpret_cast<u32x4*>(Bs + (rsub + 32 * i) * ROW + scol) = pb[i];
  };

  // K position of B inside its segment (elements) and the segment's byte offset.
  int kin = 0;
  uint32_t segoff = 0;
  const int kseg = static_cast<int>(j.kseg);
  const uint32_t segb = static_cast<uint32_t>(j.segb);
  auto next_kb = [&]() -> uint32_t {
    kin += 64;
    const bool wrap = kin == kseg;
    kin = wrap ? 0 : kin;
    segoff += wrap ? segb : 0u;
    return segoff + static_cast<uint32_t>(kin) * 2;
  };

  const int arow = wm * WTM + (lane & 31);
  const int brow = wn * WTN + (lane & 31);
  const int sw = lds_swz(lane);
  // One K chunk out of LDS stage st (4 MFMA k-steps), with the next step's fragments read
  // while the current step multiplies, and (if X is given) the prefetched chunk in X written
  // into the other stage a quarter per k-step, so the LDS writes overlap the MFMAs.
  auto compute = [&](int st, const u32x4* xa, const u32x4* xb) {
    const unsigned char* As = smem + st * STAGE;
    const unsigned char* Bs = As + BM * ROW;
    unsigned char* Ao = smem + (st ^ 1) * STAGE;
    unsigned char* Bo = Ao + BM * ROW;
    bf16x8 af[2][TM], bfr[2][TN];
    auto fread = [&](int s, int b) {
      const int phys = (((2 * s) + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int im = 0; im < TM; ++im)
        af[b][im] = *reinterpret_cast<const bf16x8*>(As + (arow + 32 * im) * ROW + phys);
#pragma unroll
      for (int jn = 0; jn < TN; ++jn)
        bfr[b][jn] = *reinterpret_cast<const bf16x8*>(Bs + (brow + 32 * jn) * ROW + phys);
    };
    fread(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) fread(s + 1, (s + 1) & 1);
#pragma unroll
      for (int jn = 0; jn < TN; ++jn)
#pragma unroll
        for (int im = 0; im < TM; ++im)
          acc[jn][im] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[s & 1][jn], af[s & 1][im],
                                                                acc[jn][im], 0, 0, 0);
      if (xa) {
#pragma unroll
        for (int i = s * ACH / 4; i < (s + 1) * ACH / 4; ++i)
          *reinterpret_cast<u32x4*>(Ao + (rsub + 32 * i) * ROW + scol) = xa[i];
#pragma unroll
        for (int i = s * BCH / 4; i < (s + 1) * BCH / 4; ++i)
          *reinterpret_cast<u32x4*>(Bo + (rsub + 32 * i) * ROW + scol) = xb[i];
      }
    }
  };

  // K is a multiple of 128 here, so the chunk count KT is even: the loop runs chunk pairs
  // with no control flow inside, and the last pair is peeled.  Invariant at the top of a
  // half-iteration: the current stage holds chunk c, one register set holds chunk c+1
  // (in flight or arrived), the other set is free and receives chunk c+2.
  const int KT = j.K / 64;
  gload(pa0, pb0, 0, 0);
  gload(pa1, pb1, ROW, next_kb());
  sstore(pa0, pb0, 0);
  __syncthreads();
  for (int kt = 0; kt + 2 < KT; kt += 2) {
    gload(pa0, pb0, static_cast<uint32_t>(kt + 2) * ROW, next_kb());
    compute(0, pa1, pb1);
    sched_chunk<TM * TN, TM + TN, ACH + BCH, ACH + BCH>();
    __syncthreads();
    gload(pa1, pb1, static_cast<uint32_t>(kt + 3) * ROW, next_kb());
    compute(1, pa0, pb0);
    sched_chunk<TM * TN, TM + TN, ACH + BCH, ACH + BCH>();
    __syncthreads();
  }
  compute(0, pa1, pb1);
  sched_chunk<TM * TN, TM + TN, 0, ACH + BCH>();
  __syncthreads();
  compute(1, nullptr, nullptr);

  // D[feature][token]: lane owns token (lane & 31) of each token tile and features
  // 8 (r / 4) + 4 (lane / 32) + (r % 4) of each feature tile.
#pragma unroll
  for (int im = 0; im < TM; ++im) {
    const int tok = wm * WTM + 32 * im + (lane & 31);
    if (tok < j.nrows) {
      char* crow = j.C + static_cast<int64_t>(tok) * j.ldc;
#pragma unroll
      for (int jn = 0; jn < TN; ++jn) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int f = wn * WTN + 32 * jn + 8 * qd + 4 * (lane >> 5);
          u32x2 pk;
          pk[0] = pack_bf16x2(act_fn<ACT>(acc[jn][im][4 * qd + 0]),
                              act_fn<ACT>(acc[jn][im][4 * qd + 1]));
          pk[1] = pack_bf16x2(act_fn<ACT>(acc[jn][im][4 * qd + 2]),
                              act_fn<ACT>(acc[jn][im][4 * qd + 3]));
          *reinterpret_cast<u32x2*>(crow + f * 2) = pk;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs g) {
  constexpr int BM = 64, BN = 64, BK = 16, LDSW = 68;
  __shared__ __attribute__((aligned(16))) float As[BK][LDSW];
  __shared__ __attribute__((aligned(16))) float Bs[BK][LDSW];
  Job j;
  if (!decode_tile<BM, BN, 4>(g, j)) return;
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  const int lr = t >> 2, lc = (t & 3) * 4;
  const int ar = lr < j.rows_left ? lr : j.rows_left - 1;
  const char* ap = j.A + static_cast<int64_t>(ar) * j.lda + lc * 4;
  const char* bp = j.B + static_cast<int64_t>(lr) * j.ldb + lc * 4;
  float acc[4][4] = {};
  for (int kt = 0; kt < j.K / BK; ++kt) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(ap + static_cast<int64_t>(kt) * BK * 4);
    const f32x4 bv = *reinterpret_cast<const f32x4*>(bp + bseg_offset(j, kt * BK, 4));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      As[lc + q][lr] = av[q];
      Bs[lc + q][lr] = bv[q];
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
    if (r < j.nrows) {
      f32x4 o;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) o[jj] = apply_act(acc[i][jj], j.act);
      *reinterpret_cast<f32x4*>(j.C + static_cast<int64_t>(r) * j.ldc + tx * 16) = o;
    }
  }
}

int grid_of(const GemmArgs& a, int BN) {
  int64_t total = static_cast<int64_t>(a.p0.max_tiles) * (a.p0.N / BN);
  if (a.nprob > 1) total += static_cast<int64_t>(a.p1.max_tiles) * (a.p1.N / BN);
  return static_cast<int>(total);
}

}  // namespace

int gemm_block_m(int dtype) { return dtype == 1 ? 256 : 64; }

int gemm_block_n(int dtype, int n0, int n1) {
  if (dtype != 1) return 64;
  return (n0 % 256 == 0 && n1 % 256 == 0) ? 256 : 128;
}

hipError_t launch_expert_gemm(const GemmArgs& a, hipStream_t s) {
  const int BN = gemm_block_n(a.dtype, a.p0.N, a.nprob > 1 ? a.p1.N : a.p0.N);
  const int grid = grid_of(a, BN);
  if (grid == 0) return hipSuccess;
  const int act = a.p0.act;  // both problems of one launch share the activation
  if (a.dtype == 1) {
#define MOE_GEMM_LAUNCH(BNV, ACTV) \
  hipLaunchKernelGGL((gemm_bf16_kernel<256, BNV, ACTV>), dim3(grid), dim3(kThreads), 0, s, a)
    if (BN == 256) {
      if (act == 0) MOE_GEMM_LAUNCH(256, 0);
      else if (act == 1) MOE_GEMM_LAUNCH(256, 1);
      else MOE_GEMM_LAUNCH(256, 2);
    } else {
      if (act == 0) MOE_GEMM_LAUNCH(128, 0);
      else if (act == 1) MOE_GEMM_LAUNCH(128, 1);
      else MOE_GEMM_LAUNCH(128, 2);
    }
#undef MOE_GEMM_LAUNCH
  } else {
    hipLaunchKernelGGL(gemm_f32_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
