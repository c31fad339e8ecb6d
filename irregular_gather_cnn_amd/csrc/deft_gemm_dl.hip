// bf16 MFMA GEMMs of the deformable convolution layer with direct
// global-to-LDS staging (gfx950).
//
// The three contractions of the layer (DefT explainer page, "The argument in
// one glance": the main convolution stays a GEMM; its backward adds dCol and
// dW) stream the 2-byte column matrix through HBM, so at the layer's shapes
// they are bound by memory bandwidth as much as by the matrix cores.  This
// kernel keeps both sides busy:
//   * operands go from HBM/L2 straight into LDS with buffer loads that write
//     LDS (no register round trip), four 32-deep k stages in flight;
//   * a buffer resource bounds every load, so rows, columns and k beyond the
//     operand read as zero (out-of-range offsets are set to 0x80000000);
//   * an operand stored k-contiguous ("row" form) is staged as 64-byte rows
//     and read with ds_read_b128; an operand stored contiguous along m or n
//     ("k-major" form, e.g. dY [Cout][pixels] or the columns seen from dW) is
//     staged as it lies and turned into MFMA fragments by ds_read_b64_tr_b16,
//     so no transpose pass over HBM is needed;
//   * 16-byte chunks are XOR-swizzled so fragment reads are free of bank
//     conflicts;
//   * results whose output is contiguous along m leave through LDS: each wave
//     transposes its 128x128 block there and writes whole 16-byte chunks.
// 256 threads = 2x2 waves; the tile shape, ring depth and occupancy are set
// per operation (GemmCfg): 256x256 tiles, 128x128 per wave (16 32x32x16 MFMA
// blocks), one workgroup per CU for dW; 256x128 tiles, two per CU, for dCol;
// 128x256 tiles, two per CU, with a shallower ring for the L2-resident weights,
// for the forward.
#include "deft_device.h"
#include "deft_internal.h"

namespace deft {
namespace {

constexpr int kBK = 32;  // k elements per stage (64 bytes per row)

// Tile shape of one GEMM: BM x BN per workgroup of 2 x 2 waves (each wave
// BM/2 x BN/2), STAGES-deep LDS ring (loads run STAGES-1 stages ahead), OCC
// workgroups per CU the LDS and registers are sized for.  STAGES_B < STAGES
// gives B a shallower ring of its own: for an A operand streamed from HBM and
// a B operand that stays in the L2 (the forward's weights), the LDS goes to
// keeping more of A's long-latency loads in flight.
template <int BM_, int BN_, int STAGES_, int OCC_, int STAGES_B_ = STAGES_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, STAGES = STAGES_, OCC = OCC_, STAGES_B = STAGES_B_;
  static_assert(STAGES_B >= 2 && STAGES_B <= STAGES, "B ring depth");
  static constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  static constexpr int kStageBytes = (BM + BN) * kBK * 2;  // A + B per stage
  static constexpr int kPerA = BM * kBK * 2 / 1024 / 4;     // 1 KB loads per wave per stage, A
  static constexpr int kPerB = BN * kBK * 2 / 1024 / 4;     // and B
  static constexpr int kLdsMain = (STAGES * BM + STAGES_B * BN) * kBK * 2;
  static constexpr int kEpiStride = WM * 2 + 16;            // bytes per transposed row
  static constexpr int kLdsEpi = 4 * WN * kEpiStride;
  static constexpr int kLds = kLdsMain > kLdsEpi ? kLdsMain : kLdsEpi;
};
using Cfg256 = GemmCfg<256, 256, 4, 1>;
__device__ __forceinline__ uint2 read_tr(const unsigned char* p) {
  const bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)p);
  return __builtin_bit_cast(uint2, v);
}

// Row-form swizzle (64-byte rows, 4 chunks): 16 consecutive rows reading the
// same logical chunk hit 16 distinct 16-byte bank slots.
__device__ __forceinline__ int swz_row(int r) { return (r >> 2) & 3; }
// k-major swizzle (rows of 2*ROWS bytes): the four k rows a 16-lane group of
// a transposed read touches land in four distinct 64-byte bank windows.
__device__ __forceinline__ int swz_kmaj(int k) { return 4 * (k & 3); }

// Issues the loads of one operand's stage: rows [0, ROWS) (row form) or k
// rows [0, kBK) (k-major form, ROWS columns) of the tile, `op_off` giving the
// byte offset of each 16-byte chunk or kOOB.
template <bool KMAJ, int ROWS, class F>
__device__ __forceinline__ void issue_operand(const rsrc_t r, unsigned char* base, int wave, int lane,
                                              int k0, const F& op_off) {
  constexpr int kPer = ROWS * kBK * 2 / 1024 / 4;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = wave * kPer + i;
    unsigned char* dst = base + b * 1024;
    int off;
    if constexpr (!KMAJ) {
      const int row = 16 * b + (lane >> 2);
      const int c = (lane & 3) ^ swz_row(row);
      off = op_off(row, k0 + 8 * c);
    } else {
      const int pos = b * 1024 + lane * 16;
      const int krow = pos / (2 * ROWS);
      const int c = ((pos % (2 * ROWS)) >> 4) ^ swz_kmaj(krow);
      off = op_off(k0 + krow, 8 * c);
    }
    load_lds16(r, dst, off);
  }
}

// MFMA fragment (8 consecutive k of row/column `rc` of the tile) for k-chunk
// pair `ks` (16 k) of a stage.
template <bool KMAJ, int ROWS>
__device__ __forceinline__ uint4 fragment(const unsigned char* base, int rc0, int ks, int lane) {
  if constexpr (!KMAJ) {
    const int row = rc0 + (lane & 31);
    const int c = 2 * ks + (lane >> 5);
    return *(const uint4*)(base + row * (kBK * 2) + ((c ^ swz_row(row)) << 4));
  } else {
    const int g = lane >> 4, j = lane & 15;
    const int n = rc0 + 16 * (g & 1) + 4 * (j & 3);
    const int c = n >> 3;
    uint2 h[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int krow = 16 * ks + 8 * (g >> 1) + 4 * t + (j >> 2);
      h[t] = read_tr(base + krow * (2 * ROWS) + ((c ^ swz_kmaj(krow)) << 4) + (n & 7) * 2);
    }
    return make_uint4(h[0].x, h[0].y, h[1].x, h[1].y);
  }
}

template <class Op>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Op::Cfg::OCC, Op::Cfg::OCC))) void k_gemm_dl(
    const Op op) {
  using C = typename Op::Cfg;
  constexpr int MI = C::MI, NI = C::NI, kStages = C::STAGES, kStageBytes = C::kStageBytes;
  constexpr int kIssue = C::kPerA + C::kPerB;  // loads per wave per stage
  extern __shared__ __align__(16) unsigned char smem[];
  const TileCoord tc = op.tile(blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS destinations go to M0
  const int wm = wave >> 1, wn = wave & 1;
  const rsrc_t ra = op.rsrc_a(), rb = op.rsrc_b();

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto issue = [&](int s) {
    unsigned char* st = smem + (s % kStages) * kStageBytes;
    const int k0 = tc.kb + s * kBK;
    issue_operand<Op::A_KMAJ, C::BM>(ra, st, wave, lane, k0,
                                     [&](int x, int y) { return op.a_off(tc, x, y); });
    issue_operand<Op::B_KMAJ, C::BN>(rb, st + C::BM * kBK * 2, wave, lane, k0,
                                     [&](int x, int y) { return op.b_off(tc, x, y); });
  };
  // A stage holds two 16-k steps.  The fragments of the next step are read
  // while the MFMAs of the current one run, also across the stage boundary:
  // the barrier that publishes stage it+1 sits between the two MFMA groups of
  // stage it, so its wait overlaps matrix work already queued.
  constexpr int kReads = MI * (Op::A_KMAJ ? 2 : 1) + NI * (Op::B_KMAJ ? 2 : 1);  // LDS reads per step
  auto read_step = [&](int s, int ks, uint4* fa, uint4* fb) {
    const unsigned char* a = smem + (s % kStages) * kStageBytes;
    const unsigned char* b = a + C::BM * kBK * 2;
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i] = fragment<Op::A_KMAJ, C::BM>(a, wm * C::WM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[j] = fragment<Op::B_KMAJ, C::BN>(b, wn * C::WN + j * 32, ks, lane);
  };
  auto mfma_step = [&](const uint4* fa, const uint4* fb) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                            __builtin_bit_cast(bf16x8_t, fb[j]), acc[i][j], 0, 0, 0);
  };
  // interleave the step's LDS reads with the MFMAs of the previous step
  auto interleave = [&]() {
#pragma unroll
    for (int u = 0; u < kReads; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                   // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, (MI * NI) / kReads > 0 ? (MI * NI) / kReads : 1, 0);  // MFMAs
    }
  };
  // waits until stage s has landed, given how many later stages were issued
  auto wait_stage = [&](int later) {
    if (later >= 3) wait_vm<3 * kIssue>();
    else if (later == 2) wait_vm<2 * kIssue>();
    else if (later == 1) wait_vm<kIssue>();
    else wait_vm<0>();
  };

  const int nk = (tc.ke - tc.kb + kBK - 1) / kBK;
  uint4 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
  if constexpr (C::STAGES_B < C::STAGES) {
    // Separate rings: A [SA][BM x kBK], then B [SB][BN x kBK].  Issue order:
    // A(0..SA-1), B(0..SB-1), then after the barrier of iteration j, A(j+SA)
    // and B(j+SB).  A(s) always precedes B(s), so stage s has landed once no
    // more loads are outstanding than were issued after B(s).
    constexpr int SA = C::STAGES, SB = C::STAGES_B, kA = C::kPerA, kB = C::kPerB;
    constexpr int kABytes = C::BM * kBK * 2, kBBytes = C::BN * kBK * 2;
    unsigned char* ringA = smem;
    unsigned char* ringB = smem + SA * kABytes;
    auto issueA = [&](int st) {
      issue_operand<Op::A_KMAJ, C::BM>(ra, ringA + (st % SA) * kABytes, wave, lane, tc.kb + st * kBK,
                                       [&](int x, int y) { return op.a_off(tc, x, y); });
    };
    auto issueB = [&](int st) {
      issue_operand<Op::B_KMAJ, C::BN>(rb, ringB + (st % SB) * kBBytes, wave, lane, tc.kb + st * kBK,
                                       [&](int x, int y) { return op.b_off(tc, x, y); });
    };
    auto read2 = [&](int st, int ks, uint4* fa, uint4* fb) {
      const unsigned char* a = ringA + (st % SA) * kABytes;
      const unsigned char* b = ringB + (st % SB) * kBBytes;
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = fragment<Op::A_KMAJ, C::BM>(a, wm * C::WM + i * 32, ks, lane);
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[j] = fragment<Op::B_KMAJ, C::BN>(b, wn * C::WN + j * 32, ks, lane);
    };
    // loads issued after B(st) by the end of iteration it-1
    auto after_b = [&](int st, int it) {
      int cnt = 0, j0 = st - SB + 1;
      if (st < SB) {
        cnt = kB * (min(SB, nk) - st - 1);
        j0 = 0;
      }
      const int j1 = it - 1;
      if (j1 >= j0) {
        cnt += kA * max(0, min(j1, nk - SA - 1) - j0 + 1);
        cnt += kB * max(0, min(j1, nk - SB - 1) - j0 + 1);
      }
      return cnt;
    };
#pragma unroll
    for (int st = 0; st < SA; ++st)
      if (st < nk) issueA(st);
#pragma unroll
    for (int st = 0; st < SB; ++st)
      if (st < nk) issueB(st);
    if (nk > 0) {
      wait_vm_atmost(after_b(0, 0));
      __syncthreads();
      read2(0, 0, fa0, fb0);
    }
    for (int it = 0; it < nk; ++it) {
      read2(it, 1, fa1, fb1);
      mfma_step(fa0, fb0);
      interleave();
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave is done reading stage it
      if (it + 1 < nk) {
        wait_vm_atmost(after_b(it + 1, it));
        __syncthreads();
        if (it + SA < nk) issueA(it + SA);  // into the buffers of stage it
        if (it + SB < nk) issueB(it + SB);
        read2(it + 1, 0, fa0, fb0);
      }
      mfma_step(fa1, fb1);
      interleave();
    }
  } else {
#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < nk) issue(s);
  if (nk > 0) {
    wait_stage(min(kStages - 1, nk - 1));
    __syncthreads();
    read_step(0, 0, fa0, fb0);
  }
  for (int it = 0; it < nk; ++it) {
    read_step(it, 1, fa1, fb1);
    mfma_step(fa0, fb0);
    interleave();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave is done reading stage it
    if (it + 1 < nk) {
      // stages issued after it+1 so far: up to it+STAGES-1
      wait_stage(min(kStages - 2, nk - 2 - it));
      __syncthreads();
      if (it + kStages < nk) issue(it + kStages);  // into the buffer of stage it
      read_step(it + 1, 0, fa0, fb0);
    }
    mfma_step(fa1, fb1);
    interleave();
  }
  }

  const int mw = tc.m0 + wm * C::WM, nw = tc.n0 + wn * C::WN;
  op.observe(acc, mw, nw, lane);
  if constexpr (Op::LDS_EPILOGUE) {
    // Transpose this wave's block through LDS: row n (local) holds the
    // wave's 128 m values; each lane owns 4 consecutive m of one n per block.
    __syncthreads();
    constexpr int kEpiStride = C::kEpiStride;
    unsigned char* reg = smem + wave * C::WN * kEpiStride;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int nl = j * 32 + (lane & 31);
        const float add = op.column_add(nw + nl);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ml = i * 32 + 8 * q + 4 * (lane >> 5);
          uint2 v;
          v.x = pack_bf16x2(acc[i][j][4 * q] + add, acc[i][j][4 * q + 1] + add);
          v.y = pack_bf16x2(acc[i][j][4 * q + 2] + add, acc[i][j][4 * q + 3] + add);
          *(uint2*)(reg + nl * kEpiStride + ml * 2) = v;
        }
      }
    __syncthreads();
    constexpr int kCh = C::WM / 8, kRows = 64 / kCh;  // 16-byte chunks per row, rows per pass
#pragma unroll 4
    for (int it = 0; it < C::WN / kRows; ++it) {
      const int nl = it * kRows + lane / kCh, c = lane % kCh;
      const uint4 v = *(const uint4*)(reg + nl * kEpiStride + c * 16);
      op.store_chunk(nw + nl, mw + c * 8, v);
    }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) op.store_acc(tc, mw + i * 32, nw + j * 32, acc[i][j], lane);
  }
}

__host__ __device__ inline uint32_t rsrc_bytes(size_t bytes) {
  return bytes > 0x7ffffff0u ? 0x7ffffff0u : (uint32_t)bytes;
}

// ---- forward: C[m = q][n = co] = sum_k cols[q][k] Wt[co][k]; y[img][co][p] = C + b[co] ----
template <class CfgT>
struct DlFwdT {
  using Cfg = CfgT;
  static constexpr bool A_KMAJ = false, B_KMAJ = false, LDS_EPILOGUE = true;
  const bf16_t* cols;  // [M][K]
  const bf16_t* wt;    // [N][K]
  const bf16_t* bias;  // nullable
  bf16_t* y;
  int M, N, K, HoWo, tilesM, tilesN;
  FastDiv div_howo;
  __device__ rsrc_t rsrc_a() const { return make_rsrc(cols, rsrc_bytes((size_t)M * K * 2)); }
  __device__ rsrc_t rsrc_b() const { return make_rsrc(wt, rsrc_bytes((size_t)N * K * 2)); }
  __device__ TileCoord tile(int bid) const {
    const int lb = xcd_swizzle(bid, tilesM * tilesN);
    const int mt = lb / tilesN, nt = lb - mt * tilesN;
    return TileCoord{mt * Cfg::BM, nt * Cfg::BN, 0, K, 0};
  }
  __device__ int a_off(const TileCoord& tc, int row, int k) const {
    const int m = tc.m0 + row;
    return (m < M && k < K) ? (m * K + k) * 2 : kOOB;
  }
  __device__ int b_off(const TileCoord& tc, int row, int k) const {
    const int n = tc.n0 + row;
    return (n < N && k < K) ? (n * K + k) * 2 : kOOB;
  }
  template <int MI_, int NI_>
  __device__ void observe(const f32x16_t (&)[MI_][NI_], int, int, int) const {}
  __device__ float column_add(int n) const { return (bias && n < N) ? bf16_to_f32(bias[n]) : 0.f; }
  // 8 consecutive pixels q = m..m+7 of output channel n (never split by an
  // image boundary: HoWo % 8 == 0 on this path)
  __device__ void store_chunk(int n, int m, const uint4 v) const {
    if (n >= N || m >= M) return;
    const int img = fdiv(m, div_howo), p = m - img * HoWo;
    store16_nt(y + ((size_t)img * N + n) * HoWo + p, v);
  }
  __device__ void store_acc(const TileCoord&, int, int, const f32x16_t&, int) const {}
};

// Forward tiles: 128 pixels x 256 output channels, two workgroups per CU, with
// a 2-deep ring for the L2-resident weights (84 us against 92 us for
// 256 x 256 at 50 176 pixels); shapes with fewer pixels or output channels
// take smaller tiles so the grid still covers the chip (at least 384 tiles).
using DlFwd = DlFwdT<GemmCfg<128, 256, 3, 2, 2>>;
using DlFwdMid = DlFwdT<GemmCfg<128, 128, 4, 2>>;
using DlFwdSmall = DlFwdT<GemmCfg<64, 128, 4, 2>>;

// ---- dCol: C[m = e][n = q] = sum_co W2[e][co] dY[img(q)][co][p(q)]; dcol[q][e] ----
struct DlDcol {
  using Cfg = GemmCfg<256, 128, 3, 2>;
  static constexpr bool A_KMAJ = false, B_KMAJ = true, LDS_EPILOGUE = true;
  const bf16_t* w2;  // [M][K]
  const bf16_t* dy;  // [img][K][HoWo]
  bf16_t* dcol;      // [N][M]
  uint32_t* maxbits;
  int M, N, K, HoWo, tilesM, tilesN;
  FastDiv div_howo;
  __device__ rsrc_t rsrc_a() const { return make_rsrc(w2, rsrc_bytes((size_t)M * K * 2)); }
  __device__ rsrc_t rsrc_b() const { return make_rsrc(dy, rsrc_bytes((size_t)N * K * 2)); }
  __device__ TileCoord tile(int bid) const {
    // consecutive workgroups (one XCD) share the dY tile of one pixel range
    const int lb = xcd_swizzle(bid, tilesM * tilesN);
    const int nt = lb / tilesM, mt = lb - nt * tilesM;
    return TileCoord{mt * Cfg::BM, nt * Cfg::BN, 0, K, 0};
  }
  __device__ int a_off(const TileCoord& tc, int row, int k) const {
    const int m = tc.m0 + row;
    return (m < M && k < K) ? (m * K + k) * 2 : kOOB;
  }
  // 8 consecutive pixels starting at tile column `col` of channel k
  __device__ int b_off(const TileCoord& tc, int k, int col) const {
    const int q = tc.n0 + col;
    if (k >= K || q >= N) return kOOB;
    const int img = fdiv(q, div_howo), p = q - img * HoWo;
    return ((img * K + k) * HoWo + p) * 2;
  }
  // running max of |dCol| (fp32 bits), one atomic per wave at most; skipped
  // when no maxbits word is given (only the fixed-point scatter needs it)
  template <int MI_, int NI_>
  __device__ void observe(const f32x16_t (&acc)[MI_][NI_], int mw, int nw, int lane) const {
    if (!maxbits) return;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < MI_; ++i)
#pragma unroll
      for (int j = 0; j < NI_; ++j) {
        if (nw + j * 32 + (lane & 31) >= N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mw + i * 32 + acc_row(lane, r) < M) mx = fmaxf(mx, fabsf(acc[i][j][r]));
      }
    for (int s = 1; s < 64; s <<= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
    if (lane == 0 && __float_as_uint(mx) > __hip_atomic_load(maxbits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(maxbits, __float_as_uint(mx));
  }
  __device__ float column_add(int) const { return 0.f; }
  __device__ void store_chunk(int n, int m, const uint4 v) const {
    if (n >= N || m >= M) return;
    store16_nt(dcol + (size_t)n * M + m, v);
  }
  __device__ void store_acc(const TileCoord&, int, int, const f32x16_t&, int) const {}
};

// ---- dW partial of split z: part[z][co][e] = sum_{q in split} dY[img(q)][co][p(q)] cols[q][e] ----
struct DlDw {
  using Cfg = Cfg256;
  static constexpr bool A_KMAJ = false, B_KMAJ = true, LDS_EPILOGUE = false;
  const bf16_t* dy;    // [img][M][HoWo]
  const bf16_t* cols;  // [P][N]
  float* part;         // [splits][M][N]
  int M, N, P, HoWo, tilesM, tilesN, splits, kper;
  FastDiv div_howo;
  __device__ rsrc_t rsrc_a() const { return make_rsrc(dy, rsrc_bytes((size_t)P * M * 2)); }
  __device__ rsrc_t rsrc_b() const { return make_rsrc(cols, rsrc_bytes((size_t)P * N * 2)); }
  __device__ TileCoord tile(int bid) const {
    // the tiles of one split sit together (they share its dY rows)
    const int per = tilesM * tilesN;
    const int lb = xcd_swizzle(bid, per * splits);
    const int z = lb / per, r = lb - z * per;
    const int mt = r / tilesN, nt = r - mt * tilesN;
    const int kb = z * kper, ke = min(P, kb + kper);
    return TileCoord{mt * Cfg::BM, nt * Cfg::BN, kb, ke, z};
  }
  // 8 consecutive pixels q..q+7 (one image) of output channel m
  __device__ int a_off(const TileCoord& tc, int row, int q) const {
    const int m = tc.m0 + row;
    if (m >= M || q >= tc.ke) return kOOB;
    const int img = fdiv(q, div_howo), p = q - img * HoWo;
    return ((img * M + m) * HoWo + p) * 2;
  }
  __device__ int b_off(const TileCoord& tc, int q, int col) const {
    const int e = tc.n0 + col;
    return (q < tc.ke && e < N) ? (q * N + e) * 2 : kOOB;
  }
  template <int MI_, int NI_>
  __device__ void observe(const f32x16_t (&)[MI_][NI_], int, int, int) const {}
  __device__ float column_add(int) const { return 0.f; }
  __device__ void store_chunk(int, int, const uint4) const {}
  __device__ void store_acc(const TileCoord& tc, int mb, int nb, const f32x16_t& acc, int lane) const {
    const int n = nb + (lane & 31);
    if (n >= N) return;
    float* dst = part + (size_t)tc.z * M * N;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mb + acc_row(lane, r);
      if (m < M) dst[(size_t)m * N + n] = acc[r];
    }
  }
};

template <class Op>
hipError_t run_dl(const char* name, const Op& op, int grid, hipStream_t st) {
  auto kern = k_gemm_dl<Op>;
  constexpr int lds = Op::Cfg::kLds;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  if (grid == 0) return hipSuccess;
  DEFT_LAUNCH(name, kern, dim3(grid), dim3(256), lds, st, op);
  return hipGetLastError();
}

int tiles(int x, int t) { return (x + t - 1) / t; }

}  // namespace

bool gemm_dl_supported(const deft_plan& p) {
  if (p.d.dtype != DEFT_BF16) return false;
  const size_t howo = (size_t)p.ho * p.wo, P = (size_t)p.d.n * howo;
  if (howo % 8 || p.d.c_out % 8 || p.ck % 8) return false;
  // every byte offset of every operand fits the 31-bit buffer offset
  const size_t lim = 0x7ffffff0u;
  return P * p.ck * 2 < lim && P * p.d.c_out * 2 < lim && (size_t)p.d.c_out * p.ck * 2 < lim;
}

void gemm_dl_dw_split(const deft_plan& p, int* splits, int* kper) {
  const int P = p.d.n * p.ho * p.wo;
  const int per = tiles(p.d.c_out, DlDw::Cfg::BM) * tiles(p.ck, DlDw::Cfg::BN);
  int s = 256 / per;
  if (s < 1) s = 1;
  int k = (P + s - 1) / s;
  k = (k + kBK - 1) / kBK * kBK;
  if (k < kBK) k = kBK;
  *kper = k;
  *splits = (P + k - 1) / k;
}

template <class Op>
static hipError_t dl_forward_with(const deft_plan& p, const void* wt, const void* cols, const void* b, void* y,
                                  hipStream_t st) {
  Op op;
  op.cols = (const bf16_t*)cols; op.wt = (const bf16_t*)wt; op.bias = (const bf16_t*)b; op.y = (bf16_t*)y;
  op.M = p.d.n * p.ho * p.wo; op.N = p.d.c_out; op.K = p.ck; op.HoWo = p.ho * p.wo;
  op.div_howo = make_fastdiv(op.HoWo);
  op.tilesM = tiles(op.M, Op::Cfg::BM); op.tilesN = tiles(op.N, Op::Cfg::BN);
  return run_dl("gemm_forward", op, op.tilesM * op.tilesN, st);
}

hipError_t dl_gemm_forward(const deft_plan& p, const void* wt, const void* cols, const void* b, void* y,
                           hipStream_t st) {
  const int M = p.d.n * p.ho * p.wo, N = p.d.c_out;
  auto count = [&](int bm, int bn) { return tiles(M, bm) * tiles(N, bn); };
  if (count(DlFwd::Cfg::BM, DlFwd::Cfg::BN) >= 384) return dl_forward_with<DlFwd>(p, wt, cols, b, y, st);
  if (count(DlFwdMid::Cfg::BM, DlFwdMid::Cfg::BN) >= 384) return dl_forward_with<DlFwdMid>(p, wt, cols, b, y, st);
  return dl_forward_with<DlFwdSmall>(p, wt, cols, b, y, st);
}

hipError_t dl_gemm_dcol(const deft_plan& p, const void* w2, const void* dy, void* dcol, uint32_t* maxbits,
                        hipStream_t st) {
  DlDcol op;
  op.w2 = (const bf16_t*)w2; op.dy = (const bf16_t*)dy; op.dcol = (bf16_t*)dcol; op.maxbits = maxbits;
  op.M = p.ck; op.N = p.d.n * p.ho * p.wo; op.K = p.d.c_out; op.HoWo = p.ho * p.wo;
  op.div_howo = make_fastdiv(op.HoWo);
  op.tilesM = tiles(op.M, DlDcol::Cfg::BM); op.tilesN = tiles(op.N, DlDcol::Cfg::BN);
  return run_dl("gemm_dcol", op, op.tilesM * op.tilesN, st);
}

hipError_t dl_gemm_dw(const deft_plan& p, const void* dy, const void* cols, float* part, hipStream_t st) {
  DlDw op;
  op.dy = (const bf16_t*)dy; op.cols = (const bf16_t*)cols; op.part = part;
  op.M = p.d.c_out; op.N = p.ck; op.P = p.d.n * p.ho * p.wo; op.HoWo = p.ho * p.wo;
  op.div_howo = make_fastdiv(op.HoWo);
  op.tilesM = tiles(op.M, DlDw::Cfg::BM); op.tilesN = tiles(op.N, DlDw::Cfg::BN);
  gemm_dl_dw_split(p, &op.splits, &op.kper);
  return run_dl("gemm_dw", op, op.tilesM * op.tilesN * op.splits, st);
}

}  // namespace deft
