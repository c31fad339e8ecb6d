// bf16 MFMA GEMMs of the deformable convolution layer with direct
// global-to-LDS staging (gfx950).
//
// The three contractions of the layer (DefT explainer page, "The argument in
// one glance": the main convolution stays a GEMM; its backward adds dCol and
// dW) stream the 2-byte column matrix through HBM, so at the layer's shapes
// they are bound by memory bandwidth as much as by the matrix cores.  Common
// to the kernels here:
//   * operands go from HBM/L2 straight into LDS with buffer loads that write
//     LDS (no register round trip);
//   * a buffer resource bounds every load, so rows, columns and k beyond the
//     operand read as zero (out-of-range offsets are set to 0x80000000);
//   * an operand stored k-contiguous ("row" form) is staged as rows of the
//     stage depth and read with ds_read_b128; an operand stored contiguous
//     along m or n ("k-major" form, e.g. dY [Cout][pixels] or the columns seen
//     from dW) is staged as it lies and turned into MFMA fragments by
//     ds_read_b64_tr_b16, so no transpose pass over HBM is needed;
//   * 16-byte chunks are XOR-swizzled so fragment reads are free of bank
//     conflicts;
//   * results whose output is contiguous along m leave through LDS: each wave
//     transposes its block there and writes whole 16-byte chunks.
// Kernels:
//   * k_gemm_dl: 2 x 2 waves, per-operation tile and ring (dCol; the forward
//     on shapes with few rows per CU);
//   * k_gemm_ws: 8 waves, waves 0-3 staging only A and 4-7 only B (dW);
//   * k_gemm_vd: 4 waves, one workgroup per CU with an equal share of the
//     output rows, 64-deep stages (the forward at the layer's main shapes).
#include <algorithm>

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

// Row-form swizzle, rows of 2*BK bytes (BK/8 16-byte chunks): the rows a
// 16-lane phase of a fragment read touches (16 consecutive rows, one logical
// chunk each) hit 16 distinct 16-byte slots of a 256-byte bank window.
// 64-byte rows (BK 32) put 4 rows in a window, 128-byte rows (BK 64) two.
template <int BK>
__device__ __forceinline__ int swz_row(int r) {
  static_assert(BK == 32 || BK == 64, "stage depth");
  if constexpr (BK == 32) return (r >> 2) & 3;
  else return (r >> 1) & 7;
}
// k-major swizzle (rows of 2*ROWS bytes): the four k rows a 16-lane group of
// a transposed read touches land in four distinct 64-byte bank windows.
__device__ __forceinline__ int swz_kmaj(int k) { return 4 * (k & 3); }

// Issues the loads of one operand's stage: rows [0, ROWS) (row form) or k
// rows [0, BK) (k-major form, ROWS columns) of the tile, `op_off` giving the
// byte offset of each 16-byte chunk or kOOB.  The four staging waves of the
// operand share the stage (`wave` 0..3).
template <bool KMAJ, int ROWS, int BK, class F>
__device__ __forceinline__ void issue_operand(const rsrc_t r, unsigned char* base, int wave, int lane,
                                              int k0, const F& op_off) {
  constexpr int kPer = ROWS * BK * 2 / 1024 / 4;
  constexpr int kCh = BK / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = wave * kPer + i;
    unsigned char* dst = base + b * 1024;
    int off;
    if constexpr (!KMAJ) {
      const int row = (64 / kCh) * b + lane / kCh;
      const int c = (lane % kCh) ^ swz_row<BK>(row);
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
template <bool KMAJ, int ROWS, class F>
__device__ __forceinline__ void issue_operand(const rsrc_t r, unsigned char* base, int wave, int lane,
                                              int k0, const F& op_off) {
  issue_operand<KMAJ, ROWS, kBK>(r, base, wave, lane, k0, op_off);
}

// MFMA fragment (8 consecutive k of row/column `rc` of the tile) for 16-k
// step `ks` of a stage.
template <bool KMAJ, int ROWS, int BK>
__device__ __forceinline__ uint4 fragment(const unsigned char* base, int rc0, int ks, int lane) {
  if constexpr (!KMAJ) {
    const int row = rc0 + (lane & 31);
    const int c = 2 * ks + (lane >> 5);
    return *(const uint4*)(base + row * (BK * 2) + ((c ^ swz_row<BK>(row)) << 4));
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
template <bool KMAJ, int ROWS>
__device__ __forceinline__ uint4 fragment(const unsigned char* base, int rc0, int ks, int lane) {
  return fragment<KMAJ, ROWS, kBK>(base, rc0, ks, lane);
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

// ---------------------------------------------------------------------------
// Eight-wave GEMM with operand-specialised staging.  Waves 0-3 stage only A
// and waves 4-7 only B, each operand into its own LDS ring; all eight waves
// compute, 2 x 4 of them, each a WM x WN block.  A wave's vector-memory
// counter retires its loads in issue order, so a wave that had issued both a
// far-ahead load of the HBM-streamed operand and a near load of the
// L2-resident one could not wait for the near one without also waiting for
// the far one: the streamed operand's ring depth would buy no lookahead.
// With one operand per wave, each ring's depth is that operand's lookahead.
// One workgroup per CU (two waves per SIMD).
template <int BM_, int BN_, int SA_, int SB_, int BK_ = 64>
struct WsCfg {
  static constexpr int BM = BM_, BN = BN_, SA = SA_, SB = SB_, BK = BK_;
  static constexpr int KS = BK / 16;  // 16-k MFMA steps per stage
  static constexpr int WM = BM / 2, WN = BN / 4, MI = WM / 32, NI = WN / 32;
  static constexpr int kABytes = BM * BK * 2, kBBytes = BN * BK * 2;
  static constexpr int kPerA = kABytes / 1024 / 4;  // 1 KB loads per staging wave per stage
  static constexpr int kPerB = kBBytes / 1024 / 4;
  static_assert(kPerA * 4096 == kABytes && kPerB * 4096 == kBBytes, "stage = whole 1 KB loads per wave");
  static constexpr int kLdsMain = SA * kABytes + SB * kBBytes;
  static constexpr int kEpiStride = WM * 2 + 16;  // bytes per transposed row of a wave's block
  static constexpr int kLdsEpi = 8 * WN * kEpiStride;
  static constexpr int kLds = kLdsMain > kLdsEpi ? kLdsMain : kLdsEpi;
};

template <class Op>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_ws(const Op op) {
  using C = typename Op::Cfg;
  constexpr int MI = C::MI, NI = C::NI, BK = C::BK, KS = C::KS;
  extern __shared__ __align__(16) unsigned char smem[];
  const TileCoord tc = op.tile(blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS destinations go to M0
  const int wm = wave >> 2, wn = wave & 3;
  const bool stages_a = wave < 4;
  const int lw = wave & 3;
  const rsrc_t ra = op.rsrc_a(), rb = op.rsrc_b();
  unsigned char* ringA = smem;
  unsigned char* ringB = smem + C::SA * C::kABytes;

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // this wave's operand: ring depth and loads per stage
  const int depth = stages_a ? C::SA : C::SB;
  const int per = stages_a ? C::kPerA : C::kPerB;
  auto issue = [&](int st) {
    const int k0 = tc.kb + st * BK;
    if (stages_a)
      issue_operand<Op::A_KMAJ, C::BM, BK>(ra, ringA + (st % C::SA) * C::kABytes, lw, lane, k0,
                                           [&](int x, int y) { return op.a_off(tc, x, y); });
    else
      issue_operand<Op::B_KMAJ, C::BN, BK>(rb, ringB + (st % C::SB) * C::kBBytes, lw, lane, k0,
                                           [&](int x, int y) { return op.b_off(tc, x, y); });
  };
  // row blocks of this wave that hold rows of the tile (row-balanced tiles
  // leave the last ones empty: they are neither read nor multiplied)
  const int tile_rows = min(tc.me - tc.m0, C::BM);  // me may be INT_MAX (no row limit)
  const int miv = __builtin_amdgcn_readfirstlane(max(0, min(MI, (tile_rows - wm * C::WM + 31) / 32)));
  auto read_step = [&](int st, int ks, uint4* fa, uint4* fb) {
    const unsigned char* a = ringA + (st % C::SA) * C::kABytes;
    const unsigned char* b = ringB + (st % C::SB) * C::kBBytes;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      if (i < miv) fa[i] = fragment<Op::A_KMAJ, C::BM, BK>(a, wm * C::WM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[j] = fragment<Op::B_KMAJ, C::BN, BK>(b, wn * C::WN + j * 32, ks, lane);
  };
  auto mfma_step = [&](const uint4* fa, const uint4* fb) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
      if (i < miv) {
#pragma unroll
        for (int j = 0; j < NI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                              __builtin_bit_cast(bf16x8_t, fb[j]), acc[i][j], 0, 0, 0);
      }
  };
  // interleave the next step's LDS reads with the MFMAs of the current one
  constexpr int kReads = MI * (Op::A_KMAJ ? 2 : 1) + NI * (Op::B_KMAJ ? 2 : 1);
  auto interleave = [&]() {
#pragma unroll
    for (int u = 0; u < kReads; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, (MI * NI) / kReads > 0 ? (MI * NI) / kReads : 1, 0);
    }
  };

  const int nk = (tc.ke - tc.kb + BK - 1) / BK;
  uint4 fa[2][MI], fb[2][NI];
  for (int st = 0; st < depth && st < nk; ++st) issue(st);
  if (nk > 0) {
    wait_vm_atmost(per * (min(depth, nk) - 1));  // this wave's part of stage 0 has landed
    __syncthreads();
    read_step(0, 0, fa[0], fb[0]);
  }
  // Each stage holds KS 16-k steps; the fragments of the next step are read
  // while the MFMAs of the current one run.  Before the last step of stage
  // it, the barrier that publishes stage it+1 (and frees stage it's ring
  // slots for the loads of stage it+depth) is passed while the MFMAs already
  // issued drain.
  for (int it = 0; it < nk; ++it) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) {
        read_step(it, ks + 1, fa[cur ^ 1], fb[cur ^ 1]);
        mfma_step(fa[cur], fb[cur]);
        interleave();
      } else {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave is done reading stage it
        if (it + 1 < nk) {
          // this wave's stages issued after it+1: up to it+depth-1
          wait_vm_atmost(per * max(0, min(depth - 2, nk - 2 - it)));
          __syncthreads();
          if (it + depth < nk) issue(it + depth);  // into the slot of stage it
          read_step(it + 1, 0, fa[cur ^ 1], fb[cur ^ 1]);
        }
        mfma_step(fa[cur], fb[cur]);
        interleave();
      }
    }
  }

  const int mw = tc.m0 + wm * C::WM, nw = tc.n0 + wn * C::WN;
  if constexpr (Op::LDS_EPILOGUE) {
    __syncthreads();  // the rings are free
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
    constexpr int kCh = C::WM / 8, kRows = 64 / kCh;
#pragma unroll 4
    for (int it = 0; it < C::WN / kRows; ++it) {
      const int nl = it * kRows + lane / kCh, c = lane % kCh;
      const uint4 v = *(const uint4*)(reg + nl * kEpiStride + c * 16);
      op.store_chunk(tc, nw + nl, mw + c * 8, v);
    }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) op.store_acc(tc, mw + i * 32, nw + j * 32, acc[i][j], lane);
  }
}

// ---------------------------------------------------------------------------
// Four-wave GEMM with buffer-to-LDS staging (one workgroup per CU, one wave
// per SIMD), 64-deep k stages.  A (streamed from HBM) has a 3-slot ring and
// is loaded two stages ahead, B (L2-resident) a 2-slot ring loaded one stage
// ahead; every wave stages its quarter of both.  After the barrier that
// frees the slots of stage it-1, a wave issues B(it+1) and then A(it+2), so
// before the next barrier it waits only for loads issued before B(it+1):
// the far A load never holds up the near B one (a wave's memory counter
// retires its loads in issue order).  Each wave owns all BM rows and a
// quarter of the BN columns (MI x NI 32x32 blocks, accumulators in AGPRs).
template <int BM_, int BN_>
struct VdCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, KS = 4, SA = 3, SB = 2;
  static constexpr int WM = BM, WN = BN / 4, MI = WM / 32, NI = WN / 32;
  static constexpr int kABytes = BM * BK * 2, kBBytes = BN * BK * 2;
  static constexpr int kPerA = kABytes / 1024 / 4, kPerB = kBBytes / 1024 / 4;  // 1 KB loads per wave
  static_assert(kPerA * 4096 == kABytes && kPerB * 4096 == kBBytes, "stage = whole 1 KB loads per wave");
  static_assert(BM % 32 == 0 && BN % 128 == 0, "tile");
  static constexpr int kLdsMain = SA * kABytes + SB * kBBytes;
  static constexpr int kEpiStride = WM * 2 + 16;
  static constexpr int kLdsEpi = 4 * WN * kEpiStride;
  static constexpr int kLds = kLdsMain > kLdsEpi ? kLdsMain : kLdsEpi;
};

template <class Op>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_vd(const Op op) {
  using C = typename Op::Cfg;
  constexpr int MI = C::MI, NI = C::NI, BK = C::BK, KS = C::KS, SA = C::SA, SB = C::SB;
  static_assert(!Op::A_KMAJ && !Op::B_KMAJ, "row-form operands");
  extern __shared__ __align__(16) unsigned char smem[];
  const TileCoord tc = op.tile(blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
  const rsrc_t ra = op.rsrc_a(), rb = op.rsrc_b();
  unsigned char* ringA = smem;
  unsigned char* ringB = smem + SA * C::kABytes;
  const int tile_rows = min(tc.me - tc.m0, C::BM);  // me may be INT_MAX (no row limit)

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (tc.ke - tc.kb + BK - 1) / BK;
  // Load b of a wave's share of a stage fills LDS bytes [1024 b, 1024 b +
  // 1024) of the slot: rows 8b..8b+7, lane -> row 8b + lane/8, slot chunk
  // lane%8 holding logical chunk (lane%8) ^ swz(row).  Its operand byte
  // offset is fixed up to the stage's k0, passed as the scalar offset (K is a
  // multiple of 64 here).  Every wave issues the same loads in every
  // iteration (stages past the last read zero through the range check), so
  // the waits are constant.
  constexpr int kCh = BK / 8;
  int va[C::kPerA], vb[C::kPerB];
#pragma unroll
  for (int i = 0; i < C::kPerA; ++i) {
    const int row = (64 / kCh) * (wn * C::kPerA + i) + lane / kCh;
    const int o = op.a_row(tc, row);
    va[i] = o == kOOB ? kOOB : o + 16 * ((lane % kCh) ^ swz_row<BK>(row));
  }
#pragma unroll
  for (int i = 0; i < C::kPerB; ++i) {
    const int row = (64 / kCh) * (wn * C::kPerB + i) + lane / kCh;
    const int o = op.b_row(tc, row);
    vb[i] = o == kOOB ? kOOB : o + 16 * ((lane % kCh) ^ swz_row<BK>(row));
  }
  auto soff_of = [&](int st) { return st < nk ? (tc.kb + st * BK) * 2 : 0x7fff0000; };
  const uint32_t ldsA = lds_addr_of(ringA) + wn * C::kPerA * 1024;
  const uint32_t ldsB = lds_addr_of(ringB) + wn * C::kPerB * 1024;
  auto issueA = [&](int st) {
    const uint32_t base = ldsA + (st % SA) * C::kABytes;
    const int so = soff_of(st);
#pragma unroll
    for (int i = 0; i < C::kPerA; ++i) load_lds16_so(ra, base + i * 1024, va[i], so);
  };
  auto issueB = [&](int st) {
    const uint32_t base = ldsB + (st % SB) * C::kBBytes;
    const int so = soff_of(st);
#pragma unroll
    for (int i = 0; i < C::kPerB; ++i) load_lds16_so(rb, base + i * 1024, vb[i], so);
  };
  uint4 fa[2][MI], fb[2][NI];
  // B fragments first: every MFMA of a step uses one, while the A fragment
  // of row block i is needed only from its (i*NI)-th MFMA on
  auto read_step = [&](int st, int ks, uint4* fa_, uint4* fb_) {
    const unsigned char* a = ringA + (st % SA) * C::kABytes;
    const unsigned char* b = ringB + (st % SB) * C::kBBytes;
#pragma unroll
    for (int j = 0; j < NI; ++j) fb_[j] = fragment<false, C::BN, BK>(b, wn * C::WN + j * 32, ks, lane);
#pragma unroll
    for (int i = 0; i < MI; ++i) fa_[i] = fragment<false, C::BM, BK>(a, i * 32, ks, lane);
  };
  auto mfma_step = [&](const uint4* fa_, const uint4* fb_) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa_[i]),
                                                            __builtin_bit_cast(bf16x8_t, fb_[j]), acc[i][j], 0, 0, 0);
  };
  auto interleave = [&]() {
#pragma unroll
    for (int u = 0; u < MI * NI; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (u < MI + NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  if (nk <= 0) return;  // (uniform) no k range
  // prologue: B(0), A(0), then what the barrier before iteration 0 would
  // have issued in the steady state (A(1), B(1), A(2)); stage 0 lands first
  issueB(0);
  issueA(0);
  issueA(1);
  issueB(1);
  issueA(2);
  wait_vm<2 * C::kPerA + C::kPerB>();
  __syncthreads();
  read_step(0, 0, fa[0], fb[0]);
  for (int it = 0; it < nk; ++it) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) {
        read_step(it, ks + 1, fa[cur ^ 1], fb[cur ^ 1]);
        mfma_step(fa[cur], fb[cur]);
        interleave();
      } else {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave is done reading stage it
        // stage it+1 has landed once only A(it+2), issued after B(it+1), is
        // outstanding
        wait_vm<C::kPerA>();
        __syncthreads();
        // slots of stage it are free: B(it+2) first, then A(it+3)
        issueB(it + 2);
        issueA(it + 3);
        read_step(it + 1, 0, fa[cur ^ 1], fb[cur ^ 1]);
        mfma_step(fa[cur], fb[cur]);
        interleave();
      }
    }
  }
  wait_vm<0>();  // the out-of-range tail loads

  const int mw = tc.m0, nw = tc.n0 + wn * C::WN;
  if constexpr (Op::LDS_EPILOGUE) {
    __syncthreads();  // the rings are free
    constexpr int kEpiStride = C::kEpiStride;
    unsigned char* reg = smem + wn * C::WN * kEpiStride;
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
    constexpr int kCh = C::WM / 8, kRows = 64 / kCh;
#pragma unroll 4
    for (int it = 0; it < (C::WN + kRows - 1) / kRows; ++it) {
      const int nl = it * kRows + lane / kCh, c = lane % kCh;
      // kCh need not divide 64, nor kRows WN
      if (lane < kRows * kCh && nl < C::WN && c * 8 < tile_rows) {
        const uint4 v = *(const uint4*)(reg + nl * kEpiStride + c * 16);
        op.store_chunk(tc, nw + nl, mw + c * 8, v);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) op.store_acc(tc, mw + i * 32, nw + j * 32, acc[i][j], lane);
  }
}

template <class Op>
hipError_t run_vd(const char* name, const Op& op, int grid, hipStream_t st) {
  auto kern = k_gemm_vd<Op>;
  constexpr int lds = Op::Cfg::kLds;
  static_assert(lds <= 160 * 1024, "LDS");
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  if (grid == 0) return hipSuccess;
  DEFT_LAUNCH(name, kern, dim3(grid), dim3(256), lds, st, op);
  return hipGetLastError();
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

// Forward with the rows balanced over one workgroup per CU: the M = N*Ho*Wo
// output rows are split into whole 8-row units, each workgroup taking an
// equal contiguous share (at most 256 rows; MFMA blocks past its share read
// zero rows and are not stored), all output channels in 256-wide column
// tiles.  Every CU then streams the same number of column rows, where
// 128-row tiles left some CUs with two tiles and others with one.
template <class CfgT>
struct FwdBalT {
  using Cfg = CfgT;
  static constexpr bool A_KMAJ = false, B_KMAJ = false, LDS_EPILOGUE = true;
  const bf16_t* cols;  // [M][K]
  const bf16_t* wt;    // [N][K]
  const bf16_t* bias;  // nullable
  bf16_t* y;
  int M, N, K, HoWo, gm, gn, units;
  FastDiv div_howo;
  __device__ rsrc_t rsrc_a() const { return make_rsrc(cols, rsrc_bytes((size_t)M * K * 2)); }
  __device__ rsrc_t rsrc_b() const { return make_rsrc(wt, rsrc_bytes((size_t)N * K * 2)); }
  __device__ TileCoord tile(int bid) const {
    // the column tiles of one row range sit on one XCD (they share its rows)
    const int lb = xcd_swizzle(bid, gm * gn);
    const int mr = lb / gn, nt = lb - mr * gn;
    const int u0 = (int)((long long)mr * units / gm), u1 = (int)((long long)(mr + 1) * units / gm);
    TileCoord t{8 * u0, nt * Cfg::BN, 0, K, 0};
    t.me = 8 * u1;
    return t;
  }
  __device__ int a_off(const TileCoord& tc, int row, int k) const {
    const int m = tc.m0 + row;
    return (m < tc.me && k < K) ? (m * K + k) * 2 : kOOB;
  }
  // byte offset of row `row` of the tile's A (B) rows, or kOOB
  __device__ int a_row(const TileCoord& tc, int row) const {
    const int m = tc.m0 + row;
    return m < tc.me ? m * K * 2 : kOOB;
  }
  __device__ int b_row(const TileCoord& tc, int row) const {
    const int n = tc.n0 + row;
    return n < N ? n * K * 2 : kOOB;
  }
  __device__ int b_off(const TileCoord& tc, int row, int k) const {
    const int n = tc.n0 + row;
    return (n < N && k < K) ? (n * K + k) * 2 : kOOB;
  }
  __device__ float column_add(int n) const { return (bias && n < N) ? bf16_to_f32(bias[n]) : 0.f; }
  // 8 consecutive pixels q = m..m+7 of output channel n (never split by an
  // image boundary: HoWo % 8 == 0 on this path)
  __device__ void store_chunk(const TileCoord& tc, int n, int m, const uint4 v) const {
    if (n >= N || m >= tc.me) return;
    const int img = fdiv(m, div_howo), p = m - img * HoWo;
    store16_nt(y + ((size_t)img * N + n) * HoWo + p, v);
  }
  __device__ void store_acc(const TileCoord&, int, int, const f32x16_t&, int) const {}
};

using FwdVd = FwdBalT<VdCfg<224, 256>>;
// the same kernel for shares of at most 192, 160, 128 or 64 rows
using FwdVd192 = FwdBalT<VdCfg<192, 256>>;
using FwdVd160 = FwdBalT<VdCfg<160, 256>>;
using FwdVdMid = FwdBalT<VdCfg<128, 256>>;
using FwdVdSmall = FwdBalT<VdCfg<64, 256>>;

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
          if (mw + i * 32 + acc_row(lane, r) < M) {
            const float a = fabsf(acc[i][j][r]);
            if (a <= 3.402823466e38f) mx = fmaxf(mx, a);  // NaN and Inf are flagged by the scatter instead
          }
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

// ---- dCol with the weight block resident in LDS ----
// dcol[q][e] = sum_co W2[e][co] dY[img(q)][co][p(q)] for K = Cout = 256.  The
// 256 x 256 block of W2 that a workgroup's rows need (128 KB) is loaded once
// and stays in LDS; only dY streams, through a 4-stage ring that runs on
// across the workgroup's pixel tiles, so a CU receives its W2 block once
// instead of once per output tile.  A workgroup owns one 256-row block of e
// and a contiguous range of 128-pixel tiles; the 9 workgroups that share a
// pixel range (and so its dY) are consecutive after the XCD swizzle.  Eight
// waves, 4 (e) x 2 (pixels), each 64 x 64 of the tile.
//
// Between tiles the ring doubles as the epilogue's transpose buffer (4 KB a
// wave): each wave leaves its block as 32-pixel passes of whole 128-byte
// rows, eight rows per store instruction.  So that the ring is free then,
// the next tile's first three dY stages are loaded into registers during the
// last three stages of the current one and written into the ring after the
// epilogue.  Every wave issues the same loads and stores in every tile
// (out-of-range ones carry an offset past the buffer), and vector-memory
// operations retire in issue order here, so the wait counts are constants.
struct DcolRes {
  static constexpr int BM = 256, BN = 128, K = 256, BK = 32, SL = K / BK;  // SL stages (W2 slices) per tile
  static constexpr int RING = 4, kSlice = BM * BK * 2, kStage = BK * BN * 2;
  static constexpr int kLds = SL * kSlice + RING * kStage;  // 128 KB + 32 KB
  const bf16_t* w2;  // [M][K]
  const bf16_t* dy;  // [img][K][HoWo]
  bf16_t* dcol;      // [N][M]
  int M, N, HoWo, nrb, groups, tilesN;
  FastDiv div_howo;
};
static_assert(DcolRes::kLds <= 160 * 1024, "LDS");
static_assert(DcolRes::SL == 8 && DcolRes::RING == 4, "the stage schedule below assumes 8 stages and 4 slots");

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_dcol_res(const DcolRes p) {
  using C = DcolRes;
  constexpr int K = C::K, BK = C::BK, SL = C::SL;
  typedef unsigned v4u32_t __attribute__((ext_vector_type(4)));
  constexpr int kNt = 2;  // non-temporal stores: the sampling backward reads dCol next, from HBM
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* wblk = smem;                   // [SL][BM rows][BK] row form, rows of 64 bytes
  unsigned char* ring = smem + SL * C::kSlice;  // [RING][BK k rows][BN] k-major
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int lb = xcd_swizzle(blockIdx.x, p.nrb * p.groups);
  const int grp = lb / p.nrb, rb = lb - grp * p.nrb;
  const int t0 = (int)((long long)p.tilesN * grp / p.groups), t1 = (int)((long long)p.tilesN * (grp + 1) / p.groups);
  const int e0 = rb * C::BM;
  if (t1 <= t0) return;  // (uniform)
  const rsrc_t rw = make_rsrc(p.w2, rsrc_bytes((size_t)p.M * K * 2));
  const rsrc_t rd = make_rsrc(p.dy, rsrc_bytes((size_t)p.N * K * 2));
  const __amdgpu_buffer_rsrc_t rdb = make_brsrc(p.dy, rsrc_bytes((size_t)p.N * K * 2));
  const __amdgpu_buffer_rsrc_t rc = make_brsrc(p.dcol, (uint32_t)((size_t)p.N * p.M * 2));

  // W2 slice s (k in [32 s, 32 s + 32)): 16 loads of 1 KB, two per wave; load
  // b covers rows 16 b .. 16 b + 15, lane -> row 16 b + lane / 4, slot chunk
  // lane % 4 holding logical chunk (lane % 4) ^ swz(row)
  int wofs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = wave * 2 + i, row = 16 * b + lane / 4;
    wofs[i] = ((e0 + row) * K + 8 * ((lane % 4) ^ swz_row<BK>(row))) * 2;
  }
  const uint32_t wlds = lds_addr_of(wblk) + wave * 2 * 1024;
  auto issue_w = [&](int s) {
#pragma unroll
    for (int i = 0; i < 2; ++i) load_lds16_so(rw, wlds + s * C::kSlice + i * 1024, wofs[i], s * BK * 2);
  };
  // dY stage (32 k rows x 128 pixels): the 1 KB share of `wave` holds k rows
  // 4 wave .. 4 wave + 3, lane -> k row 4 wave + lane / 16, slot chunk lane %
  // 16 holding the 8 pixels of logical chunk (lane % 16) ^ swz_kmaj(k row)
  const int krow = 4 * wave + lane / 16;
  const int dchunk = (lane % 16) ^ swz_kmaj(krow);
  const uint32_t dlds = lds_addr_of(ring) + wave * 1024;
  int dbase = kOOB;  // byte offset of (k row krow, the lane's 8 pixels) of the tile being loaded
  auto set_tile = [&](int t) {
    const int q = t * C::BN + 8 * dchunk;
    if (t < t1 && q < p.N) {
      const int img = fdiv(q, p.div_howo), pp = q - img * p.HoWo;
      dbase = ((img * K + krow) * p.HoWo + pp) * 2;
    } else {
      dbase = kOOB;
    }
  };
  auto issue_d = [&](int s) {  // stage s of the tile being loaded, into slot s % 4
    load_lds16_so(rd, dlds + (s % C::RING) * C::kStage, dbase, s * BK * p.HoWo * 2);
  };

  // prologue: W0 D0 W1 D1 W2 D2 W3..W7 (the first tile waits slice by slice)
  set_tile(t0);
  issue_w(0);
  issue_d(0);
  issue_w(1);
  issue_d(1);
  issue_w(2);
  issue_d(2);
#pragma unroll
  for (int s = 3; s < SL; ++s) issue_w(s);

  f32x16_t acc[2][2];
  uint4 rnext[3];  // stages 0..2 of the next tile, loaded during stages 5..7
  unsigned char* epi = ring + wave * 4096;  // this wave's transpose buffer: 32 pixels x 128 bytes
  const int ntile = t1 - t0;
  for (int t = 0; t < ntile; ++t) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
    for (int s = 0; s < SL; ++s) {
      // Operations issued after stage s's dY load.  First tile: W slices and
      // dY stages as in the prologue, then the two younger loads.  Later
      // tiles: stages 0..2 came through registers (no wait); from stage 3 on
      // the two younger loads.
      if (s == 0) { if (t == 0) wait_vm<16>(); }
      else if (s == 1) { if (t == 0) wait_vm<14>(); }
      else if (s == 2) { if (t == 0) wait_vm<12>(); }
      else wait_vm<2>();
      __syncthreads();  // stage s visible to all; the slot read in stage s - 1 is free
      if (s + 3 < SL) {
        issue_d(s + 3);
      } else {
        if (s + 3 == SL) set_tile(t0 + t + 1);
        const int u = s + 3 - SL;
        rnext[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rdb, dbase, u * BK * p.HoWo * 2, 0));
      }
      const unsigned char* a = wblk + s * C::kSlice;
      const unsigned char* b = ring + (s % C::RING) * C::kStage;
      uint4 fa[2][2], fb[2][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[ks][i] = fragment<false, C::BM, BK>(a, wm * 64 + i * 32, ks, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[ks][j] = fragment<true, C::BN, BK>(b, wn * 64 + j * 32, ks, lane);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[ks][i]),
                                                                __builtin_bit_cast(bf16x8_t, fb[ks][j]), acc[i][j], 0, 0,
                                                                0);
    }
    // Epilogue of tile t.  A lane of a 32 x 32 block holds 4 consecutive e of
    // one pixel per register group; trading lanes 32..63 of one group with
    // lanes 0..31 of the next gives each lane 8 consecutive e (16 bytes).
    // Chunks are XOR-swizzled by (row / 2) % 8 so the writes of 16 rows hit
    // distinct banks.
    __syncthreads();  // every wave is done with the ring
    const int n0 = (t0 + t) * C::BN + wn * 64, half = lane >> 5, row = lane & 31;
    const int ew = e0 + wm * 64;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // register groups 2h (rows +0..3) and 2h + 1 (rows +8..11)
          const f32x16_t& v = acc[i][j];
          const uint32_t ylo = pack_bf16x2(v[8 * h + 0], v[8 * h + 1]), yhi = pack_bf16x2(v[8 * h + 2], v[8 * h + 3]);
          const uint32_t xlo = pack_bf16x2(v[8 * h + 4], v[8 * h + 5]), xhi = pack_bf16x2(v[8 * h + 6], v[8 * h + 7]);
          const auto sl = __builtin_amdgcn_permlane32_swap(ylo, xlo, false, false);
          const auto sh = __builtin_amdgcn_permlane32_swap(yhi, xhi, false, false);
          const int c = 4 * i + 2 * h + half;  // 16-byte chunk of the 128-byte row
          *(uint4*)(epi + row * 128 + ((c ^ ((row >> 1) & 7)) << 4)) = make_uint4(sl[0], sh[0], sl[1], sh[1]);
        }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int qr = 8 * u + lane / 8, c = lane % 8;
        const uint4 w = *(const uint4*)(epi + qr * 128 + ((c ^ ((qr >> 1) & 7)) << 4));
        const int q = n0 + 32 * j + qr;
        const v4u32_t val = {w.x, w.y, w.z, w.w};
        __builtin_amdgcn_raw_buffer_store_b128(val, rc, q < p.N ? (q * p.M + ew + 8 * c) * 2 : kOOB, 0, kNt);
      }
    }
    __syncthreads();  // the transpose buffers are read
    if (t + 1 < ntile) {
#pragma unroll
      for (int u = 0; u < 3; ++u) *(uint4*)(ring + u * C::kStage + wave * 1024 + lane * 16) = rnext[u];
    }
  }
  wait_vm<0>();  // the out-of-range tail loads have landed before the workgroup ends
}

// ---- dW partial of split z: part[z][co][e] = sum_{q in split} dY[img(q)][co][p(q)] cols[q][e] ----
template <class CfgT>
struct DlDwT {
  using Cfg = CfgT;
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
hipError_t run_ws(const char* name, const Op& op, int grid, hipStream_t st) {
  auto kern = k_gemm_ws<Op>;
  constexpr int lds = Op::Cfg::kLds;
  static_assert(lds <= 160 * 1024, "LDS");
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  if (grid == 0) return hipSuccess;
  DEFT_LAUNCH(name, kern, dim3(grid), dim3(512), lds, st, op);
  return hipGetLastError();
}

// dW on the eight-wave kernel: dY (L2 / Infinity Cache, read by the 9 column
// tiles of each split) is staged by waves 0-3, the columns (HBM) by waves
// 4-7, four stages deep each.
using DlDw = DlDwT<Cfg256>;
using DwWs = DlDwT<WsCfg<256, 256, 4, 4, 32>>;

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
  const int per = tiles(p.d.c_out, DwWs::Cfg::BM) * tiles(p.ck, DwWs::Cfg::BN);
  int s = p.cus / per;
  if (s < 1) s = 1;
  int k = (P + s - 1) / s;
  constexpr int bk = DwWs::Cfg::BK;
  k = (k + bk - 1) / bk * bk;
  if (k < bk) k = bk;
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
  // Row-balanced four-wave kernel: one workgroup per CU, each an equal share
  // of whole 8-row units and 256 output channels, in the instance with the
  // smallest row tile that holds the share (it computes every row block of
  // its tile); k in whole 64-deep stages.  More rows than one round of
  // 224-row shares holds run in as many rounds as needed, each CU taking one
  // share per round.  Shares of fewer than 32 rows go to the tiled kernels.
  {
    const int units = M / 8, gn = tiles(N, FwdVd::Cfg::BN);
    const int slots = (p.cus + gn - 1) / gn;  // row ranges per round
    const int rounds = std::max(1, tiles(units, slots * (FwdVd::Cfg::BM / 8)));
    const int gm = std::min(units, rounds * slots);
    if (p.ck % FwdVd::Cfg::BK == 0 && gm > 0) {
      const int smax = 8 * ((units + gm - 1) / gm), smin = 8 * (units / gm);
      auto run = [&](auto op) {
        op.cols = (const bf16_t*)cols; op.wt = (const bf16_t*)wt; op.bias = (const bf16_t*)b; op.y = (bf16_t*)y;
        op.M = M; op.N = N; op.K = p.ck; op.HoWo = p.ho * p.wo;
        op.div_howo = make_fastdiv(op.HoWo);
        op.units = units; op.gn = gn; op.gm = gm;
        return run_vd("gemm_forward", op, gm * gn, st);
      };
      if (smax > FwdVd192::Cfg::BM) return run(FwdVd());
      if (smax > FwdVd160::Cfg::BM) return run(FwdVd192());
      if (smax > FwdVdMid::Cfg::BM) return run(FwdVd160());
      if (smax > FwdVdSmall::Cfg::BM) {
        if (smin >= 64) return run(FwdVdMid());
      } else if (smin >= 32) {
        return run(FwdVdSmall());
      }
    }
  }
  auto count = [&](int bm, int bn) { return tiles(M, bm) * tiles(N, bn); };
  if (count(DlFwd::Cfg::BM, DlFwd::Cfg::BN) >= 384) return dl_forward_with<DlFwd>(p, wt, cols, b, y, st);
  if (count(DlFwdMid::Cfg::BM, DlFwdMid::Cfg::BN) >= 384) return dl_forward_with<DlFwdMid>(p, wt, cols, b, y, st);
  return dl_forward_with<DlFwdSmall>(p, wt, cols, b, y, st);
}

hipError_t dl_gemm_dcol(const deft_plan& p, const void* w2, const void* dy, void* dcol, uint32_t* maxbits,
                        hipStream_t st) {
  const int M = p.ck, N = p.d.n * p.ho * p.wo;
  if (!maxbits && p.d.c_out == DcolRes::K && M % DcolRes::BM == 0) {
    DcolRes op;
    op.w2 = (const bf16_t*)w2; op.dy = (const bf16_t*)dy; op.dcol = (bf16_t*)dcol;
    op.M = M; op.N = N; op.HoWo = p.ho * p.wo; op.div_howo = make_fastdiv(op.HoWo);
    op.nrb = M / DcolRes::BM; op.tilesN = tiles(N, DcolRes::BN);
    op.groups = std::max(1, std::min(op.tilesN, p.cus / op.nrb));
    constexpr int lds = DcolRes::kLds;
    hipError_t e = hipFuncSetAttribute((const void*)k_dcol_res, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    DEFT_LAUNCH("gemm_dcol", k_dcol_res, dim3(op.nrb * op.groups), dim3(512), lds, st, op);
    return hipGetLastError();
  }
  DlDcol op;
  op.w2 = (const bf16_t*)w2; op.dy = (const bf16_t*)dy; op.dcol = (bf16_t*)dcol; op.maxbits = maxbits;
  op.M = p.ck; op.N = p.d.n * p.ho * p.wo; op.K = p.d.c_out; op.HoWo = p.ho * p.wo;
  op.div_howo = make_fastdiv(op.HoWo);
  op.tilesM = tiles(op.M, DlDcol::Cfg::BM); op.tilesN = tiles(op.N, DlDcol::Cfg::BN);
  return run_dl("gemm_dcol", op, op.tilesM * op.tilesN, st);
}

hipError_t dl_gemm_dw(const deft_plan& p, const void* dy, const void* cols, float* part, hipStream_t st) {
  DwWs op;
  op.dy = (const bf16_t*)dy; op.cols = (const bf16_t*)cols; op.part = part;
  op.M = p.d.c_out; op.N = p.ck; op.P = p.d.n * p.ho * p.wo; op.HoWo = p.ho * p.wo;
  op.div_howo = make_fastdiv(op.HoWo);
  op.tilesM = tiles(op.M, DwWs::Cfg::BM); op.tilesN = tiles(op.N, DwWs::Cfg::BN);
  op.splits = p.dw_splits;  // the plan sized the partials' workspace for these
  op.kper = p.dw_kper;
  return run_ws("gemm_dw", op, op.tilesM * op.tilesN * op.splits, st);
}

}  // namespace deft
