// Backward pass of the deformable convolution layer for gfx950.
//
// The DefT explainer page speaks of training time only ("The argument in one
// glance", "This paper's idea"), so the backward is the exact derivative of
// the forward.  dCol = W^T dY and the pixel-range partials of dW = dY Col
// run on the MFMA GEMMs (deft_gemm.hip, deft_gemm_dl.hip); this file holds
//   k_prep_backward -- one launch: per (core tile of input pixels, offset
//                     group) the list of (output pixel, tap) pairs whose
//                     corners touch the core within the halo, in candidate
//                     order; dY sums for db; W2 / W_off^T layouts; zeroing.
//   k_sample_bwd_mf -- bf16, per (core, group, 64- or 32-channel chunk): dX
//                     of the core as MFMA products of sparse bilinear-weight
//                     tiles with the listed entries' dCol rows, each wave
//                     owning a 32 x 32 block of it, written once; the unique
//                     owner of each pair reduces dOffset over the chunk's
//                     channels into that chunk's partial.
//   k_sample_bwd   -- the same without MFMA (fp32, small chunks): lanes =
//                     channels scatter dCol x weight into a fixed-point LDS
//                     copy of the core with integer LDS atomics (order-
//                     independent sums).
//   k_sample_bwd_miss -- dOffset of every (pixel, tap) pair: the owning
//                     core's chunk partials summed in chunk order, zero for a
//                     fully outside tap; the rare taps beyond the halo
//                     computed from global memory, their dX added with global
//                     atomics; per-block dOffset sums for db_off.
//   k_woff_bwd     -- per (image, 32-channel slice, band of output rows):
//                     dW_off partials = dOffset rows against the plain
//                     patches of x, both staged in LDS, on MFMA.
//   k_dx_final     -- per 64 input pixels x 256 channels: dX_offset, the
//                     transposed offset convolution (MFMA), plus the sampling
//                     part of dX; rounded once.
//   k_reduce_final -- one fixed-order reduction of all partials to dW,
//                     dW_off, db, db_off.
// Global atomics are avoided on every hot path: on gfx950 they run far below
// the bandwidth of plain stores.
#include <algorithm>
#include <type_traits>

#include "deft_device.h"
#include "deft_internal.h"

namespace deft {

hipError_t launch_gemm_dcol(const deft_plan& p, const void* w2, const void* dy, void* dcol, uint32_t* maxbits,
                            hipStream_t st);
hipError_t launch_gemm_dw(const deft_plan& p, const void* dy, const void* cols, float* dwpart, hipStream_t st);

struct BwdParams {
  int N, Cin, H, W, Ho, Wo, KH, KW, SH, SW, PH, PW, DH, DW, G, Cg, K2, Oc, Ck;
  int CH, CW, bt_h, bt_w, halo, CC, num_wg, list_cap, capbits, xstr, dcstr;
  int lds_dx, lds_dc, lds_cnt;
  const void* x;
  const float* off;
  const void* dcol;
  const uint32_t* maxbits;  // max |dcol| as fp32 bits
  float* dxs;    // [N][H][W][Cin] fp32 (channel-minor): the sampling part of dX
  float* doffp;  // [Cg/CC][N][Oc][Ho][Wo] per-chunk dOffset partials of the pairs a core owns
  float* doff;   // [N][Oc][Ho][Wo] dOffset, written by k_sample_bwd_miss
  bf16_t* doff16;  // the same rounded to bf16 (bf16 layers), or null
  float* bpart;  // bias partials: [Cout][N] (dY sums), then [Oc][N][ceil(Ho*Wo/256)] (dOffset sums)
  int Cout;
  int4* lists;   // [num_tg][list_cap]: one list per (core, group)
  int* counts;   // [num_tg]: entries in each list
  int num_tg;    // cores x groups
  const bf16_t* xh;  // channel-minor copy of x left by a direct-gather forward, or null
};

__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
// float -> int32 rounded to nearest (halves up), one instruction
__device__ __forceinline__ int cvt_rpi(float x) {
  int r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ int ceil_div(int a, int b) { return -floor_div(-a, b); }
// acc + sum over the eight bf16 pairs of a and b (products exact in fp32)
__device__ __forceinline__ float dot2_bf16(const uint4 a, const uint4 b, float acc) {
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a.x), __builtin_bit_cast(b2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a.y), __builtin_bit_cast(b2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a.z), __builtin_bit_cast(b2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a.w), __builtin_bit_cast(b2_t, b.w), acc, false);
  return acc;
}
// Pins four 16-byte values as whole register quads (no code): the 16-byte
// LDS reads that produced them are not split into 4-byte reads.
__device__ __forceinline__ void keep_whole(uint4& a, uint4& b, uint4& c, uint4& d) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  u32x4 va = __builtin_bit_cast(u32x4, a), vb = __builtin_bit_cast(u32x4, b);
  u32x4 vc = __builtin_bit_cast(u32x4, c), vd = __builtin_bit_cast(u32x4, d);
  asm volatile("" : "+v"(va), "+v"(vb), "+v"(vc), "+v"(vd));
  a = __builtin_bit_cast(uint4, va); b = __builtin_bit_cast(uint4, vb);
  c = __builtin_bit_cast(uint4, vc); d = __builtin_bit_cast(uint4, vd);
}
// the same from zero: the first pair on the three-operand form with a zero
// addend, so no accumulator register is cleared first
__device__ __forceinline__ float dot2_bf16_0(const uint4 a, const uint4 b) {
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  float acc;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a.x), "v"(b.x));
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a.y), __builtin_bit_cast(b2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a.z), __builtin_bit_cast(b2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a.w), __builtin_bit_cast(b2_t, b.w), acc, false);
  return acc;
}

// dOffset of a block's owned entries (each (pixel, tap) pair has exactly one
// owner core): lanes = entries (lane & 31), the two lane halves take the two
// halves of the chunk's channels; dst holds the entries' dCol rows, xl the
// staged input region around the core.
template <typename T>
__device__ __forceinline__ void doffset_owned(const int4 cur, int nb, int lane, const T* dst, int dcstr, const T* xl,
                                              int xstr, int XW, int CC, int HoWo, float* doffp) {
  constexpr bool kWide = sizeof(T) == 4;
  const int r = lane & 31, half = lane >> 5;
  const int ex = __shfl(cur.x, r), ey = __shfl(cur.y, r), ez = __shfl(cur.z, r), ew = __shfl(cur.w, r);
  const uint32_t info = (uint32_t)ey;
  const bool own = r < nb && (int)info < 0;
  float gy = 0.f, gx = 0.f;
  if (own) {
    const int cy = (info >> 16) & 255, cx = (info >> 24) & 127;
    const float ly = __int_as_float(ez), lx = __int_as_float(ew);
    const float hy = 1.0f - ly, hx = 1.0f - lx;
    const T* drow = dst + r * dcstr;
    const T* b0 = xl + (cy * XW + cx) * xstr;
    const T* b1 = b0 + xstr;
    const T* b2 = b0 + XW * xstr;
    const T* b3 = b2 + xstr;
    const int hc = CC >> 1;
    if constexpr (kWide) {
      for (int cc = half * hc; cc < (half + 1) * hc; cc += 8) {
        float gv[8], v00[8], v01[8], v10[8], v11[8];
        lds_read8(drow + cc, gv);
        lds_read8(b0 + cc, v00);
        lds_read8(b1 + cc, v01);
        lds_read8(b2 + cc, v10);
        lds_read8(b3 + cc, v11);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          gy = __builtin_fmaf(gv[k], hx * (v10[k] - v00[k]) + lx * (v11[k] - v01[k]), gy);
          gx = __builtin_fmaf(gv[k], hy * (v01[k] - v00[k]) + ly * (v11[k] - v10[k]), gx);
        }
      }
    } else {
      // bf16: the four corner dot products D_q = sum_c dCol_c x_q,c on
      // the packed two-channel dot instruction (products exact in fp32),
      // then gy = hx (D10 - D00) + lx (D11 - D01), gx likewise
      float d00 = 0.f, d01 = 0.f, d10 = 0.f, d11 = 0.f;
      for (int cc = half * hc; cc < (half + 1) * hc; cc += 8) {
        const uint4 gq = *(const uint4*)(drow + cc);
        const uint4 q00 = *(const uint4*)(b0 + cc), q01 = *(const uint4*)(b1 + cc);
        const uint4 q10 = *(const uint4*)(b2 + cc), q11 = *(const uint4*)(b3 + cc);
        d00 = dot2_bf16(gq, q00, d00);
        d01 = dot2_bf16(gq, q01, d01);
        d10 = dot2_bf16(gq, q10, d10);
        d11 = dot2_bf16(gq, q11, d11);
      }
      gy = hx * (d10 - d00) + lx * (d11 - d01);
      gx = hy * (d01 - d00) + ly * (d11 - d10);
    }
  }
  gy += __shfl_xor(gy, 32);
  gx += __shfl_xor(gx, 32);
  if (own && half == 0) {
    const int t = info & 255;
    doffp[(size_t)(2 * t) * HoWo + ex] = gy;
    doffp[(size_t)(2 * t + 1) * HoWo + ex] = gx;
  }
}

// The (output pixel, tap) pairs whose corners touch one core tile of input
// pixels (for one offset group), written to that core's list; shared by the
// core's channel-chunk workgroups of the sampling backward.  One 256-thread
// workgroup per (core, group), the first num_tg workgroups of the
// backward's preparation launch: the candidates (for every tap, the output
// pixels whose tap grid point lies within halo+1 above/left and halo
// below/right of the core, where a corner can touch it) are evaluated four
// per thread per round, all loads of a round in flight together.  The kept
// pairs are compacted in candidate order (ballots and one prefix over the
// workgroup's waves per round), so a list, and everything summed in its
// order, is the same on every run.
__device__ __forceinline__ void bwd_lists_body(const BwdParams& p, int bid) {
  constexpr int NW = 4;  // waves
  constexpr int NT = 64 * NW;
  constexpr int U = 8;   // candidates per thread per round
  __shared__ int rlo_h[48], rlo_w[48], rnw[48], rsz[48], rmax;
  __shared__ uint32_t rdiv[96];
  __shared__ int wcnt[2][U * NW];  // per round parity: kept pairs per (step u, wave)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tg = xcd_swizzle(bid, p.num_tg);
  const int tile = tg / p.G, g = tg - tile * p.G;
  const int tpi = p.bt_h * p.bt_w;
  const int n = tile / tpi, trem = tile - n * tpi;
  const int Y0 = (trem / p.bt_w) * p.CH, X0 = (trem % p.bt_w) * p.CW;
  const int chn = min(p.CH, p.H - Y0), cwn = min(p.CW, p.W - X0);
  const int obase = 2 * g * p.K2;
  const int HoWo = p.Ho * p.Wo;
  int4* list = p.lists + (size_t)tg * p.list_cap;
  const float* __restrict__ offn = p.off + ((size_t)n * p.Oc + obase) * HoWo;

  // per tap: first output row / column of the candidate rectangle, its
  // width (as a divisor) and size; candidates are numbered t*R + k with R
  // the largest rectangle, so a candidate's tap is one division away
  if (tid < p.K2) {
    const int t = tid;
    const int ti = t / p.KW, tj = t - ti * p.KW;
    const int ho_lo = max(0, ceil_div(Y0 - 1 - p.halo + p.PH - ti * p.DH, p.SH));
    const int ho_hi = min(p.Ho - 1, floor_div(Y0 + chn - 1 + p.halo + p.PH - ti * p.DH, p.SH));
    const int wo_lo = max(0, ceil_div(X0 - 1 - p.halo + p.PW - tj * p.DW, p.SW));
    const int wo_hi = min(p.Wo - 1, floor_div(X0 + cwn - 1 + p.halo + p.PW - tj * p.DW, p.SW));
    const int nh = max(0, ho_hi - ho_lo + 1), nw = max(0, wo_hi - wo_lo + 1);
    rlo_h[t] = ho_lo; rlo_w[t] = wo_lo; rnw[t] = nw > 0 ? nw : 1;
    const FastDiv fd = make_fastdiv(nw > 0 ? nw : 1);
    rdiv[2 * t] = fd.m; rdiv[2 * t + 1] = fd.s;
    rsz[t] = nh * nw;
  }
  __syncthreads();
  if (tid == 0) {
    int m = 1;
    for (int t = 0; t < p.K2; ++t) m = max(m, rsz[t]);
    rmax = m;
  }
  __syncthreads();
  const int R = rmax;
  const FastDiv dR = make_fastdiv(R);
  const int ncand = p.K2 * R;
  int running = 0;  // pairs kept in earlier rounds
  for (int e0 = 0, round = 0; e0 < ncand; e0 += U * NT, ++round) {
    float dyv[U], dxv[U];
    int tt[U], pp[U], hh[U], ww[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * NT + tid;
      tt[u] = -1;
      dyv[u] = dxv[u] = 0.f;
      pp[u] = hh[u] = ww[u] = 0;
      const int t = fdiv(e, dR), k = e - t * R;
      if (e < ncand && k < rsz[t]) {
        const FastDiv fd{rdiv[2 * t], rdiv[2 * t + 1]};
        const int kr = fdiv(k, fd);
        const int ho = rlo_h[t] + kr, wo = rlo_w[t] + (k - kr * rnw[t]);
        tt[u] = t;
        hh[u] = ho; ww[u] = wo;
        pp[u] = ho * p.Wo + wo;
        dyv[u] = offn[(size_t)(2 * t) * HoWo + pp[u]];
        dxv[u] = offn[(size_t)(2 * t + 1) * HoWo + pp[u]];
      }
    }
    int4 ent[U];
    unsigned long long keep[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tt[u];
      bool k = false;
      ent[u] = make_int4(0, 0, 0, 0);
      if (t >= 0) {
        const int ti = t / p.KW, tj = t - ti * p.KW;
        const int by = hh[u] * p.SH - p.PH + ti * p.DH, bx = ww[u] * p.SW - p.PW + tj * p.DW;
        const TapIndex ix = tap_index(by, bx, dyv[u], dxv[u], p.H, p.W);
        if (!ix.outside && max(abs(ix.y0 - by), abs(ix.x0 - bx)) <= p.halo) {
          uint32_t cm = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int cy = ix.y0 + (q >> 1), cx = ix.x0 + (q & 1);
            if (cy >= Y0 && cy < Y0 + chn && cx >= X0 && cx < X0 + cwn) cm |= 1u << q;
          }
          if (cm) {
            const int oy = max(ix.y0, 0), ox = max(ix.x0, 0);
            const uint32_t owned = (oy >= Y0 && oy < Y0 + chn && ox >= X0 && ox < X0 + cwn) ? 1u : 0u;
            ent[u] = make_int4(pp[u], (int)((uint32_t)t | (cm << 9) | (owned << 31) |
                                            ((uint32_t)(ix.y0 - Y0 + 1) << 16) | ((uint32_t)(ix.x0 - X0 + 1) << 24)),
                               __float_as_int(ix.ly), __float_as_int(ix.lx));
            k = true;
          }
        }
      }
      keep[u] = __builtin_amdgcn_ballot_w64(k);
    }
    // slots in candidate order: step u, then wave, then lane
    int* wc = wcnt[round & 1];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (lane == 0) wc[u * NW + wave] = __builtin_popcountll(keep[u]);
    __syncthreads();
    // lanes of every wave: inclusive prefix over the U x NW counts
    int c = lane < U * NW ? wc[lane] : 0;
#pragma unroll
    for (int s = 1; s < U * NW; s <<= 1) {
      const int o = __shfl_up(c, s);
      if (lane >= s) c += o;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = u * NW + wave;
      const int base = running + __shfl(c, idx) - wc[idx];
      if ((keep[u] >> lane) & 1ull) list[base + __builtin_popcountll(keep[u] & below)] = ent[u];
    }
    running += __shfl(c, U * NW - 1);
  }
  // the last block of the sampling backward's MFMA form ends on a multiple
  // of 64 entries: the slots up to there hold entries with no corner and no
  // owner whose dCol row (pixel Ho*Wo) lies past the image's rows
  for (int i = running + tid; i < ((running + 63) & ~63); i += NT) list[i] = make_int4(HoWo, 0, 0, 0);
  if (tid == 0) p.counts[tg] = running;
}

// Corner q of a tap: (y0 + (q >> 1), x0 + (q & 1)), the order of tap_weights.
template <typename T>
__global__ __launch_bounds__(256) void k_sample_bwd(const BwdParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // one workgroup per (core tile, offset group, channel chunk): the chunks
  // of one core are neighbours in the XCD-aware order and share its offsets
  const int lw = xcd_swizzle(blockIdx.x, p.num_wg);
  const int nchunks = p.Cg / p.CC;
  const int tg = lw / nchunks, chunk = lw - tg * nchunks;
  const int tile = tg / p.G, g = tg - tile * p.G;
  const int tpi = p.bt_h * p.bt_w;
  const int n = tile / tpi, trem = tile - n * tpi;
  const int Y0 = (trem / p.bt_w) * p.CH, X0 = (trem % p.bt_w) * p.CW;
  const int chn = min(p.CH, p.H - Y0), cwn = min(p.CW, p.W - X0);
  const int obase = 2 * g * p.K2;
  const int HoWo = p.Ho * p.Wo;
  T* xl = (T*)smem;  // [(CH+2)*(CW+2)][xstr]: rows Y0-1..Y0+CH, cols X0-1..X0+CW
  const int4* list = p.lists + (size_t)tg * p.list_cap;
  const T* __restrict__ x = (const T*)p.x;
  const T* __restrict__ dcol = (const T*)p.dcol;

  const int L = p.counts[tg];

  // ---- per channel chunk: stage, scatter, dOffset, write the core ----
  // dX is accumulated in fixed point with integer LDS atomics (fast on this
  // LDS, unlike float atomics; integer sums do not depend on the order of the
  // atomics).  Every contribution |w*g| <= max|g| < 2^e and a (pixel,
  // channel) receives at most list_cap < 2^capbits of them.  fp32: 64-bit
  // accumulators, scale 2^S with S = 61 - capbits - e, a contribution split
  // as hi*2^32 + lo with |hi| < 2^30, exact to 2^-S.  bf16: 32-bit
  // accumulators, S = 30 - capbits - e, each contribution rounded to the
  // nearest multiple of 2^-S (relative to the sum of the contributions'
  // magnitudes the error stays below 2^-(30-capbits), far inside bf16's).
  constexpr bool kWide = sizeof(T) == 4;
  typedef typename std::conditional<kWide, unsigned long long, uint32_t>::type acc_t;
  const uint32_t gb = *p.maxbits;
  const int e = max((int)((gb >> 23) & 255u) - 126, -100);
  const int S = (kWide ? 61 : 30) - p.capbits - e;
  const float sc = ldexpf(1.0f, kWide ? S - 32 : S);
  const double inv = ldexp(1.0, -S);
  // Each wave walks blocks of BLK list entries: the block's dCol rows are
  // copied into a wave-private LDS buffer with 16-byte loads (the next
  // block's rows are already in flight in registers), then processed one
  // entry at a time with lanes = channels.
  constexpr int BLK = 32;
  constexpr int VEC = Elem<T>::VEC;
  constexpr int KQ = BLK / VEC;  // loads per lane per block, at most
  const int XW = p.CW + 2;
  const int c = lane;  // channel within the chunk (lanes >= CC idle)
  const bool act = c < p.CC;
  const size_t HW = (size_t)p.H * p.W;
  T* dst = (T*)(smem + p.lds_dc) + (size_t)wave * BLK * p.dcstr;
  acc_t* dxl = (acc_t*)(smem + p.lds_dx);  // [CH*CW][CC], then one spill slot per lane
  acc_t* spill = dxl + p.CH * p.CW * p.CC + lane;
  // Non-finite contributions (a NaN or infinite dCol) cannot be held in fixed
  // point: each sets a flag of its element instead, four bits per element
  // (1 NaN, 2 +Inf, 4 -Inf), eight elements per word, after the spill slots.
  // The element is then written as the IEEE sum of those contributions
  // would be: NaN if any was NaN or both infinities occurred, else the
  // infinity.
  uint32_t* nflags = (uint32_t*)(dxl + p.CH * p.CW * p.CC + 64);
  auto flag_nonfinite = [&](int el, float v) {
    const uint32_t f = v != v ? 1u : (v > 0.f ? 2u : 4u);
    atomicOr(nflags + (el >> 3), f << (4 * (el & 7)));
  };
  const int lpe = p.CC / VEC;  // lanes per dCol row (16-byte pieces)
  const int epi = 64 / lpe;    // rows per load instruction
  const size_t pstride = (size_t)p.N * p.Oc * HoWo;
  const FastDiv drh = make_fastdiv(p.CH + 2);
  const StageGeom sg = stage_geom<T>(p.W, X0 - 1, XW, (size_t)p.Cin * HW);
  {
    const int c0 = chunk * p.CC;
    const int cglob = g * p.Cg + c0;
    float* doffp = p.doffp + (size_t)(c0 / p.CC) * pstride + ((size_t)n * p.Oc + obase) * HoWo;
    __syncthreads();
    stage_region<T>(xl, x, p.Cin, p.H, p.W, n, cglob, p.CC, Y0 - 1, X0 - 1, p.CH + 2, XW, drh, sg, p.xstr);
    for (int k = tid; k < p.CH * p.CW * p.CC; k += 256) dxl[k] = 0;
    for (int k = tid; k < (p.CH * p.CW * p.CC + 7) / 8; k += 256) nflags[k] = 0;
    __syncthreads();
    int eb = wave * BLK;
    int4 my = make_int4(0, 0, 0, 0);
    uint4 q[KQ];
    auto load_block = [&](int b0) {
      const int nb = min(BLK, L - b0);
      my = lane < nb ? list[b0 + lane] : make_int4(0, 0, 0, 0);
#pragma unroll
      for (int k = 0; k < KQ; ++k) {
        const int r = k * epi + lane / lpe, v = lane % lpe;
        const int pix = __shfl(my.x, r & 63), t = __shfl(my.y, r & 63) & 255;
        q[k] = make_uint4(0, 0, 0, 0);
        if (k * epi < BLK && r < nb)
          q[k] = *(const uint4*)(dcol + ((size_t)n * HoWo + pix) * p.Ck + (size_t)t * p.Cin + cglob + v * VEC);
      }
    };
    if (eb < L) load_block(eb);
    for (; eb < L; eb += 4 * BLK) {
      const int nb = min(BLK, L - eb);
#pragma unroll
      for (int k = 0; k < KQ; ++k) {
        const int r = k * epi + lane / lpe, v = lane % lpe;
        if (k * epi < BLK && r < nb) *(uint4*)(dst + r * p.dcstr + v * VEC) = q[k];
      }
      const int4 cur = my;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (eb + 4 * BLK < L) load_block(eb + 4 * BLK);
      // scatter: lanes = channels.  bf16: eight entries per step, their dCol
      // values read from LDS together; every corner issues its atomic, and
      // corners outside the core add into a per-lane spill slot (lanes beyond
      // the chunk add zero), so the step has no branches.
      const int nbs = __builtin_amdgcn_readfirstlane(nb);
      if constexpr (kWide) {
        for (int r = 0; r < nbs; ++r) {
          const uint32_t info = (uint32_t)__builtin_amdgcn_readlane(cur.y, r);
          const uint32_t cm = (info >> 9) & 15u;
          const int cy = (info >> 16) & 255, cx = (info >> 24) & 127;  // corner (y0, x0) relative to (Y0-1, X0-1)
          TapIndex ix;
          ix.outside = false;
          ix.ly = __int_as_float(__builtin_amdgcn_readlane(cur.z, r));
          ix.lx = __int_as_float(__builtin_amdgcn_readlane(cur.w, r));
          float w[4];
          tap_weights(ix, w);
          if (act) {
            const float gs = Elem<T>::to_f32(dst[r * p.dcstr + c]) * sc;
            acc_t* d0 = dxl + ((cy - 1) * p.CW + (cx - 1)) * p.CC + c;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              if (cm & (1u << qq)) {
                const float xv = gs * w[qq];
                const int off = ((qq >> 1) * p.CW + (qq & 1)) * p.CC;
                if (!(fabsf(xv) <= 3.402823466e38f)) {
                  flag_nonfinite((int)(d0 + off - dxl), xv);
                  continue;
                }
                const float fh = floorf(xv);
                const uint32_t lo = (uint32_t)((xv - fh) * 4294967296.0f);
                atomicAdd(d0 + off, ((unsigned long long)(uint32_t)(int)fh << 32) | lo);
              }
            }
          }
        }
      } else {
        const int cr = min(c, p.CC - 1);
        const float scl = act ? sc : 0.f;
        for (int r0 = 0; r0 < nbs; r0 += 8) {
          float gs[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) gs[u] = Elem<T>::to_f32(dst[min(r0 + u, nbs - 1) * p.dcstr + cr]) * scl;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int r = r0 + u;
            if (r >= nbs) break;
            const uint32_t info = (uint32_t)__builtin_amdgcn_readlane(cur.y, r);
            const uint32_t cm = (info >> 9) & 15u;
            const int cy = (info >> 16) & 255, cx = (info >> 24) & 127;
            TapIndex ix;
            ix.outside = false;
            ix.ly = __int_as_float(__builtin_amdgcn_readlane(cur.z, r));
            ix.lx = __int_as_float(__builtin_amdgcn_readlane(cur.w, r));
            float w[4];
            tap_weights(ix, w);
            acc_t* d0 = dxl + ((cy - 1) * p.CW + (cx - 1)) * p.CC + c;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              acc_t* da = ((cm >> qq) & 1u) ? d0 + ((qq >> 1) * p.CW + (qq & 1)) * p.CC : spill;
              const float xv = gs[u] * w[qq];
              if (!(fabsf(xv) <= 3.402823466e38f)) {  // rare: flagged, and the fixed-point add is skipped
                if (da != spill) flag_nonfinite((int)(da - dxl), xv);
                continue;
              }
              atomicAdd(da, (uint32_t)cvt_rpi(xv));
            }
          }
        }
      }
      doffset_owned<T>(cur, nb, lane, dst, p.dcstr, xl, p.xstr, XW, p.CC, HoWo, doffp);
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    for (int k = tid; k < p.CC * chn * cwn; k += 256) {
      const int r = k / p.CC, cc = k - r * p.CC;
      const int y = r / cwn, xx = r - y * cwn;
      const int el = (y * p.CW + xx) * p.CC + cc;
      const acc_t a = dxl[el];
      const double sv = kWide ? (double)(long long)a : (double)(int)(uint32_t)a;
      float v = (float)(sv * inv);
      const uint32_t f = (nflags[el >> 3] >> (4 * (el & 7))) & 15u;
      if (f) v = ((f & 1u) || (f & 6u) == 6u) ? __builtin_nanf("") : ((f & 2u) ? __builtin_inff() : -__builtin_inff());
      p.dxs[((size_t)n * HW + (size_t)(Y0 + y) * p.W + X0 + xx) * p.Cin + cglob + cc] = v;
    }
  }
}

// One DPP row shift: lane i of each 16-lane row reads lane i - N of the row.
template <int N>
__device__ __forceinline__ float row_shr(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x110 + N, 0xf, 0xf, true));
}

// bf16 sampling backward with the scatter on the MFMA units.  The core's list
// is walked in blocks of BLK entries (BLK = 2048 / CC: 32 entries for a
// 64-channel chunk, 64 for a 32-channel one).  Lane (entry, piece) of a block
// loads 16 bytes (8 channels) of the entry's dCol row, two blocks before it is
// used (the list entries four blocks before), and with them
//   - computes the entry's offset gradient over those 8 channels (the four
//     corner dot products on the packed bf16 dot instruction, exact products
//     summed in fp32), summed over the entry's lanes by row shifts; the unique
//     owner of the pair stores it as this chunk's partial;
//   - writes the piece to the block's staged dCol tile [entry][channel];
//   - for pieces 0..3, writes the bilinear weight of corner q = piece to the
//     block's weight tile A [core pixel][entry] (the fp32 weight split into
//     bf16 hi + lo, two MFMAs, so the weights keep 16 significant bits), after
//     clearing the weight it wrote into that tile two blocks before.
// After one barrier, wave w multiplies the rows of A of its 32-pixel half with
// the staged columns of its 32-channel half (a 32-channel chunk: the two wave
// pairs take the two halves of the block's entries instead, added in a fixed
// order at the end): dX[pixel][channel] += A B in fp32 registers.  The tiles
// are double-buffered, so one barrier per block suffices.  Each wave owns its
// output block and writes it once, from the registers, into the channel-minor
// fp32 dX [N][H][W][Cin].
//
// A non-finite dCol value would reach every pixel of the core through the
// zero weights (0 x NaN = NaN).  A lane whose partial offset gradient is not
// finite (a non-finite dCol value always makes it so) records instead, for
// each non-finite value and each corner of the entry inside the core, the
// class of the product (NaN, +Inf or -Inf) in 4-bit LDS flags and stages a
// zero in its place; the write-out adds the flagged value.
template <int CC>
__global__ __launch_bounds__(256) void k_sample_bwd_mf(const BwdParams p) {
  constexpr int PPE = CC / 8;        // lanes (16-byte pieces) per list entry
  constexpr int BLK = 256 / PPE;     // list entries per block
  constexpr int KS = BLK / 16;       // MFMA k-steps per block
  constexpr int KSPLIT = 64 / CC;    // wave pairs sharing an output block
  constexpr int ROWB = BLK * 2;      // bytes per weight-tile row
  constexpr int NCH = BLK / 8;       // 16-byte chunks per weight-tile row
  constexpr int RP = 128 / BLK;      // weight-tile rows per 256 bytes (the swizzle period)
  constexpr int TILE = 64 * ROWB;    // one weight tile (hi or lo)
  constexpr int STG = BLK * CC * 2;  // one staged dCol tile
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lw = xcd_swizzle(blockIdx.x, p.num_wg);
  const int nchunks = p.Cg / CC;
  const int tg = lw / nchunks, chunk = lw - tg * nchunks;
  const int tile = tg / p.G, g = tg - tile * p.G;
  const int tpi = p.bt_h * p.bt_w;
  const int n = tile / tpi, trem = tile - n * tpi;
  const int Y0 = (trem / p.bt_w) * p.CH, X0 = (trem % p.bt_w) * p.CW;
  const int chn = min(p.CH, p.H - Y0), cwn = min(p.CW, p.W - X0);
  const int HoWo = p.Ho * p.Wo;
  const int XW = p.CW + 2;
  const int PX = p.CH * p.CW;
  const int cglob = g * p.Cg + chunk * CC;
  const int L = p.counts[tg];
  const int nblk = (L + BLK - 1) / BLK;
  const int4* __restrict__ list = p.lists + (size_t)tg * p.list_cap;
  const bf16_t* __restrict__ dcol = (const bf16_t*)p.dcol + (size_t)n * HoWo * p.Ck + cglob;
  float* doffp = p.doffp + (size_t)chunk * p.N * p.Oc * HoWo + ((size_t)n * p.Oc + 2 * g * p.K2) * HoWo;
  bf16_t* xl = (bf16_t*)smem;                     // [(CH+2)*(CW+2)][CC]: rows Y0-1..Y0+CH, cols X0-1..X0+CW
  unsigned char* wtile = smem + p.lds_dx;         // [2 buffers][hi, lo][64 pixels][BLK entries] bf16
  unsigned char* stg = smem + p.lds_dc;           // [2 buffers][BLK entries][CC channels] bf16
  uint32_t* nfl = (uint32_t*)(smem + p.lds_cnt);  // [64 pixels][CC] 4-bit flags, then an "any flag" word
  constexpr int NFW = 64 * CC / 8;

  const int e = tid / PPE, v = tid % PPE;  // this lane's entry in a block and 8-channel piece
  // Every load and store of the block loop is issued by every lane: the
  // list's last block is filled up with entries that have no corner and no
  // owner and whose dCol rows lie past the buffer's range (read as zeros),
  // blocks past the list (loaded ahead, never used) read zero entries, and
  // stores of lanes with nothing to store go past their buffer's range,
  // where they are dropped.  The loop then has no branches around memory operations, and
  // the waits for the loads in flight stay exact.
  const __amdgpu_buffer_rsrc_t lrs = make_brsrc(list, (uint32_t)((L + 63) & ~63) * 16u);
  const __amdgpu_buffer_rsrc_t drs = make_brsrc(dcol, (uint32_t)((size_t)HoWo * p.Ck * 2));
  const __amdgpu_buffer_rsrc_t ors = make_brsrc(doffp, (uint32_t)(2 * p.K2 * HoWo * 4));
  auto load_entry = [&](int b) {
    return __builtin_bit_cast(int4, __builtin_amdgcn_raw_buffer_load_b128(lrs, (b * BLK + e) * 16, 0, 0));
  };
  // dCol row of (output pixel, tap): (pix*K2 + tap)*Cin within the image
  auto load_piece = [&](int b, const int4 en) {
    const int off = ((en.x * p.K2 + (en.y & 255)) * p.Cin + v * 8) * 2;
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(drs, off, 0, 0));
  };

  // the input region around the core (read by the offset gradient): from the
  // channel-minor copy of x with buffer-to-LDS loads, else staged from x
  if (p.xh) {
    const int HWi = p.H * p.W;
    const rsrc_t xr = make_rsrc(p.xh + (size_t)n * (HWi + 1) * p.Cin, (uint32_t)((size_t)(HWi + 1) * p.Cin * 2));
    const int nslots = (p.CH + 2) * XW * PPE;
    for (int s0 = wave * 64; s0 < nslots; s0 += 256) {
      const int sl = s0 + lane, px = sl / PPE, pc = sl - px * PPE;
      const int ry = px / XW, rx = px - ry * XW;
      const int y = Y0 - 1 + ry, xx = X0 - 1 + rx;
      const int pix = ((unsigned)y < (unsigned)p.H && (unsigned)xx < (unsigned)p.W) ? y * p.W + xx : HWi;
      if (sl < nslots) load_lds16(xr, (unsigned char*)xl + s0 * 16, (pix * p.Cin + cglob + pc * 8) * 2);
    }
  } else {
    const size_t HW = (size_t)p.H * p.W;
    const FastDiv drh = make_fastdiv(p.CH + 2);
    const StageGeom sg = stage_geom<bf16_t>(p.W, X0 - 1, XW, (size_t)p.Cin * HW);
    stage_region<bf16_t>(xl, (const bf16_t*)p.x, p.Cin, p.H, p.W, n, cglob, CC, Y0 - 1, X0 - 1, p.CH + 2, XW, drh, sg,
                         CC);
  }
  // ring slots: list entries of blocks b..b+3, dCol pieces of blocks b, b+1
  int4 e0 = load_entry(0), e1 = load_entry(1), e2 = load_entry(2), e3 = load_entry(3);
  uint4 d0 = load_piece(0, e0), d1 = load_piece(1, e1);
  for (int i = tid; i < 4 * TILE / 16; i += 256) ((uint4*)wtile)[i] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i <= NFW; i += 256) nfl[i] = 0u;
  // vmcnt(0) as the builtin, so that the compiler's own waits in the loop
  // below know that nothing from here is still in flight
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();

  const int ph = wave & 1;                      // pixel half of the MFMA output block
  const int chh = KSPLIT == 1 ? wave >> 1 : 0;  // channel half
  const int kh = KSPLIT == 2 ? wave >> 1 : 0;   // half of the block's entries (32-channel chunks)
  const int arow = ph * 32 + (lane & 31);
  const int gq = lane >> 4, j16 = lane & 15;
  const int bcol = chh * 32 + 16 * (gq & 1) + 4 * (j16 & 3);
  // this lane's staged piece: 64-channel rows have their pieces swizzled by
  // bit 1 of the row, so the transposed reads of four rows hit distinct banks
  const int swz = CC == 64 ? (e & 2) : 0;
  const int soff = e * (CC * 2) + ((v ^ swz) << 4);
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // weight-tile byte offset of this lane's entry column in row 0, and of its
  // corner's core pixel relative to cy * CW + cx
  const unsigned ecol = (unsigned)(((e >> 3) << 4) + (e & 7) * 2);
  const unsigned pcv = (unsigned)((v >> 1) * p.CW + (v & 1) - p.CW - 1);
  constexpr int WSH = RP == 4 ? 2 : 3;  // (P / RP) % NCH << 4 == (P << WSH) & ((NCH - 1) << 4)
  static_assert(RP == 4 || RP == 2, "weight-tile swizzle period");
  int w0 = (int)ecol, w1 = (int)ecol;  // the weight this lane last wrote into each weight buffer

  // One block: en, dq hold its list entry and dCol piece and are refilled
  // with those of blocks b + 4 and b + 2 (whose list entry is en2).
  auto step = [&](const int b, int4& en, uint4& dq, const int4& en2, int& wold, const int buf) {
    const uint32_t info = (uint32_t)en.y;
    const float ly = __int_as_float(en.z), lx = __int_as_float(en.w);
    const float hy = 1.0f - ly, hx = 1.0f - lx;
    const int cy = (info >> 16) & 255, cx = (info >> 24) & 127;  // corner (y0, x0) relative to (Y0-1, X0-1)

    // offset gradient over this lane's channels
    const bf16_t* c00 = xl + (cy * XW + cx) * CC + v * 8;
    uint4 x00 = *(const uint4*)c00, x01 = *(const uint4*)(c00 + CC);
    uint4 x10 = *(const uint4*)(c00 + XW * CC), x11 = *(const uint4*)(c00 + (XW + 1) * CC);
    keep_whole(x00, x01, x10, x11);
    const float d00 = dot2_bf16_0(dq, x00), d01 = dot2_bf16_0(dq, x01);
    const float d10 = dot2_bf16_0(dq, x10), d11 = dot2_bf16_0(dq, x11);
    float gy = hx * (d10 - d00) + lx * (d11 - d01);
    float gx = hy * (d01 - d00) + ly * (d11 - d10);
    // (lane masks straight from the compares: no boolean is widened to a
    // register for the ballot)
    const float gsum = fabsf(gy) + fabsf(gx);
    const unsigned long long badm = __builtin_amdgcn_fcmpf(gsum, 3.402823466e38f, 10 /* unordered or > */);
    gy += row_shr<1>(gy);
    gx += row_shr<1>(gx);
    gy += row_shr<2>(gy);
    gx += row_shr<2>(gx);
    if (PPE == 8) {
      gy += row_shr<4>(gy);
      gx += row_shr<4>(gx);
    }
    {
      const bool own = (v == PPE - 1) & ((int)info < 0);
      const int o = own ? (int)((info & 255u) * (2u * (unsigned)HoWo) + (unsigned)en.x) * 4 : kOOB;
      // (the builtin stores 32-bit integers: pass the bits; gx goes one
      // offset channel further through the scalar offset)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gy), ors, o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gx), ors, o, HoWo * 4, 0);
    }

    // non-finite dCol values: flag the products, stage zeros
    uint4 dqs = dq;
    if (badm) {
      if (!(gsum <= 3.402823466e38f)) {
        const uint32_t cm = (info >> 9) & 15u;
        uint4 keep = make_uint4(~0u, ~0u, ~0u, ~0u);
#pragma unroll 1
        for (int k = 0; k < 8; ++k) {
          const uint32_t wv = k < 4 ? (k < 2 ? dq.x : dq.y) : (k < 6 ? dq.z : dq.w);
          const float gv = bf16_to_f32((wv >> (16 * (k & 1))) & 0xffffu);
          if (fabsf(gv) <= 3.402823466e38f) continue;
#pragma unroll 1
          for (int qq = 0; qq < 4; ++qq) {
            if (!((cm >> qq) & 1u)) continue;
            const int P = (cy - 1 + (qq >> 1)) * p.CW + (cx - 1 + (qq & 1));
            const float wgt = ((qq >> 1) ? ly : hy) * ((qq & 1) ? lx : hx);
            const uint32_t code = (gv != gv || wgt == 0.f) ? 1u : (gv > 0.f ? 2u : 4u);
            atomicOr(&nfl[P * (CC / 8) + v], code << (4 * k));
          }
          const uint32_t m = ~(0xffffu << (16 * (k & 1)));
          if (k < 2) keep.x &= m; else if (k < 4) keep.y &= m; else if (k < 6) keep.z &= m; else keep.w &= m;
        }
        dqs = make_uint4(dq.x & keep.x, dq.y & keep.y, dq.z & keep.z, dq.w & keep.w);
        nfl[NFW] = 1u;
      }
    }

    // this block's tiles: the weight of corner q = v (after clearing the one
    // this lane wrote into the same buffer two blocks before), the dCol piece
    unsigned char* wb = wtile + buf * 2 * TILE;
    unsigned char* sb = stg + buf * STG;
    if (v < 4) {
      // wold is in this lane's column (entry e): a location cleared already
      // holds zero, and another corner of the entry written to it now is
      // written after this clear
      *(bf16_t*)(wb + wold) = 0;
      *(bf16_t*)(wb + TILE + wold) = 0;
      if (((info >> (9 + v)) & 1u) != 0u) {
        const unsigned P = __umul24((unsigned)cy, (unsigned)p.CW) + (unsigned)cx + pcv;
        const float w = ((v >> 1) ? ly : hy) * ((v & 1) ? lx : hx);
        const bf16_t hi = f32_to_bf16(w);
        const bf16_t lo = f32_to_bf16(w - bf16_to_f32(hi));
        // row P, 16-byte chunk (e / 8) ^ ((P / RP) % NCH), element e % 8
        wold = (int)((P * ROWB + ecol) ^ ((P << WSH) & ((NCH - 1) << 4)));
        *(bf16_t*)(wb + wold) = hi;
        *(bf16_t*)(wb + TILE + wold) = lo;
      }
    }
    *(uint4*)(sb + soff) = dqs;
    // refill the slots (their values are no longer read)
    dq = load_piece(b + 2, en2);
    en = load_entry(b + 4);
    __syncthreads();

#pragma unroll
    for (int ks = kh * (KS / KSPLIT); ks < (kh + 1) * (KS / KSPLIT); ++ks) {
      const int c = 2 * ks + (lane >> 5);
      const int aoff = arow * ROWB + ((c ^ ((arow / RP) % NCH)) << 4);
      const uint4 ahi = *(const uint4*)(wb + aoff), alo = *(const uint4*)(wb + TILE + aoff);
      uint2 h[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int krow = ks * 16 + 8 * (gq >> 1) + 4 * t + (j16 >> 2);
        const int phys = (bcol >> 3) ^ (CC == 64 ? (krow & 2) : 0);
        h[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                             (__attribute__((address_space(3))) bf16x4_t*)(
                                                 sb + krow * (CC * 2) + (phys << 4) + (bcol & 7) * 2)));
      }
      const uint4 bq = make_uint4(h[0].x, h[0].y, h[1].x, h[1].y);
      mfma_chunk(acc, ahi, bq, bf16_t());
      mfma_chunk(acc, alo, bq, bf16_t());
    }
  };
  int b = 0;
  for (; b + 4 <= nblk; b += 4) {
    step(b, e0, d0, e2, w0, 0);
    step(b + 1, e1, d1, e3, w1, 1);
    step(b + 2, e2, d0, e0, w0, 0);
    step(b + 3, e3, d1, e1, w1, 1);
  }
  if (b < nblk) step(b, e0, d0, e2, w0, 0);
  if (b + 1 < nblk) step(b + 1, e1, d1, e3, w1, 1);
  if (b + 2 < nblk) step(b + 2, e2, d0, e0, w0, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // the refills past the list

  if (KSPLIT == 2) {  // the two halves of the entries, added in a fixed order
    __syncthreads();  // every wave is done with the weight tiles
    float* red = (float*)wtile;  // [pixel half][16][64]
    if (kh == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) red[(ph * 16 + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += red[(ph * 16 + r) * 64 + lane];
  }
  if (ph * 32 >= PX) return;
  const bool anyflag = nfl[NFW] != 0u;
  const int cc = chh * 32 + (lane & 31);
  const float rcw = 1.0f / (float)p.CW;
  float* dxo = p.dxs + ((size_t)n * p.H * p.W) * p.Cin + cglob + cc;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int P = ph * 32 + acc_row(lane, r);
    const int y = (int)(((float)P + 0.5f) * rcw), x = P - y * p.CW;
    if (P >= PX || y >= chn || x >= cwn) continue;
    float val = acc[r];
    if (anyflag) {
      const uint32_t f = (nfl[P * (CC / 8) + (cc >> 3)] >> (4 * (cc & 7))) & 15u;
      if (f) val += ((f & 1u) || (f & 6u) == 6u) ? __builtin_nanf("") : ((f & 2u) ? __builtin_inff() : -__builtin_inff());
    }
    dxo[((size_t)(Y0 + y) * p.W + X0 + x) * p.Cin] = val;
  }
}

// Taps beyond the halo (need > halo, not fully outside): a workgroup scans
// 256 pixels of one (image, group, tap) plane, lane = pixel; for each miss,
// the wave (lanes = channels) computes the offset gradient from global memory
// and adds the dX contributions with global atomics.  Runs after k_sample_bwd
// has written dX.  Grid: N*G*K2 planes x ceil(Ho*Wo / 256) blocks.
template <typename T>
__global__ __launch_bounds__(256) void k_sample_bwd_miss(const BwdParams p) {
  __shared__ float red[4][2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int HoWo = p.Ho * p.Wo;
  const int bpp = (HoWo + 255) / 256;  // blocks per plane
  const int plane = blockIdx.x / bpp, blk = blockIdx.x - plane * bpp;  // uniform
  const int r2 = plane / p.K2, t = plane - r2 * p.K2;
  const int n = r2 / p.G, g = r2 - n * p.G;
  const int ti = t / p.KW, tj = t - ti * p.KW;
  const int oy = 2 * (g * p.K2 + t);  // offset channels oy (dy) and oy + 1 (dx)
  const size_t HW = (size_t)p.H * p.W;
  const size_t cstride = (size_t)p.N * p.Oc * HoWo;  // between chunk partials
  const T* __restrict__ x = (const T*)p.x;
  const T* __restrict__ dcol = (const T*)p.dcol;
  const size_t obase = ((size_t)n * p.Oc + oy) * HoWo;
  const float* __restrict__ offp = p.off + obase;
  const int wpix0 = blk * 256 + (threadIdx.x & ~63);  // first pixel of this wave
  const int pix = wpix0 + lane;
  float vy = 0.f, vx = 0.f;
  bool miss = false;
  if (pix < HoWo) {
    // the chunk partials (up to four) are loaded with the offsets, in one
    // round trip, and kept only for a pair that a core owns
    const int nch = p.Cg / p.CC;
    const float* py = p.doffp + obase + pix;
    float py4[4], px4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      py4[c] = c < nch ? py[c * cstride] : 0.f;
      px4[c] = c < nch ? py[c * cstride + HoWo] : 0.f;
    }
    const int ho = pix / p.Wo, wo = pix - ho * p.Wo;
    const int by = ho * p.SH - p.PH + ti * p.DH, bx = wo * p.SW - p.PW + tj * p.DW;
    const TapIndex ix = tap_index(by, bx, offp[pix], offp[HoWo + pix], p.H, p.W);
    miss = !ix.outside && max(abs(ix.y0 - by), abs(ix.x0 - bx)) > p.halo;
    if (!ix.outside && !miss) {
      // the owning core wrote one partial per channel chunk: summed in chunk order
      vy = py4[0];
      vx = px4[0];
#pragma unroll
      for (int c = 1; c < 4; ++c)
        if (c < nch) {
          vy += py4[c];
          vx += px4[c];
        }
      for (int c = 4; c < nch; ++c) {
        vy += py[c * cstride];
        vx += py[c * cstride + HoWo];
      }
    }
  }
  // taps beyond the halo, one at a time per wave: its lanes split the channels
  unsigned long long mask = __ballot(miss);
  while (mask) {
    const int l = __ffsll((long long)mask) - 1;
    mask &= mask - 1;
    const int mpix = wpix0 + l;
    const int ho = mpix / p.Wo, wo = mpix - ho * p.Wo;
    const int by = ho * p.SH - p.PH + ti * p.DH, bx = wo * p.SW - p.PW + tj * p.DW;
    const TapIndex ix = tap_index(by, bx, offp[mpix], offp[HoWo + mpix], p.H, p.W);
    float w[4];
    tap_weights(ix, w);
    const int y0 = ix.y0, x0 = ix.x0;
    const bool r0 = y0 >= 0, r1 = y0 + 1 < p.H, q0 = x0 >= 0, q1 = x0 + 1 < p.W;
    float gy = 0.f, gx = 0.f;
    for (int c = lane; c < p.Cg; c += 64) {
      const int cg = g * p.Cg + c;
      const float gcv = Elem<T>::to_f32(dcol[((size_t)n * HoWo + mpix) * p.Ck + (size_t)t * p.Cin + cg]);
      const T* pl = x + ((size_t)n * p.Cin + cg) * HW;
      float* dl = p.dxs + (size_t)n * HW * p.Cin + cg;  // channel-minor: pixel stride Cin
      const float v00 = (r0 && q0) ? Elem<T>::to_f32(pl[(size_t)y0 * p.W + x0]) : 0.f;
      const float v01 = (r0 && q1) ? Elem<T>::to_f32(pl[(size_t)y0 * p.W + x0 + 1]) : 0.f;
      const float v10 = (r1 && q0) ? Elem<T>::to_f32(pl[(size_t)(y0 + 1) * p.W + x0]) : 0.f;
      const float v11 = (r1 && q1) ? Elem<T>::to_f32(pl[(size_t)(y0 + 1) * p.W + x0 + 1]) : 0.f;
      if (r0 && q0) atomicAdd(dl + ((size_t)y0 * p.W + x0) * p.Cin, w[0] * gcv);
      if (r0 && q1) atomicAdd(dl + ((size_t)y0 * p.W + x0 + 1) * p.Cin, w[1] * gcv);
      if (r1 && q0) atomicAdd(dl + ((size_t)(y0 + 1) * p.W + x0) * p.Cin, w[2] * gcv);
      if (r1 && q1) atomicAdd(dl + ((size_t)(y0 + 1) * p.W + x0 + 1) * p.Cin, w[3] * gcv);
      gy += gcv * ((1.0f - ix.lx) * (v10 - v00) + ix.lx * (v11 - v01));
      gx += gcv * ((1.0f - ix.ly) * (v01 - v00) + ix.ly * (v11 - v10));
    }
    for (int s = 1; s < 64; s <<= 1) {
      gy += __shfl_xor(gy, s);
      gx += __shfl_xor(gx, s);
    }
    if (lane == l) {
      vy = gy;
      vx = gx;
    }
  }
  if (pix < HoWo) {
    p.doff[obase + pix] = vy;
    p.doff[obase + HoWo + pix] = vx;
    if (p.doff16) {
      p.doff16[obase + pix] = f32_to_bf16(vy);
      p.doff16[obase + HoWo + pix] = f32_to_bf16(vx);
    }
  }
  // this block's sums of the two offset channels: db_off partials, added in a
  // fixed order (lanes by the xor tree, then waves in order)
  float sy = vy, sx = vx;
  for (int s = 32; s > 0; s >>= 1) {
    sy += __shfl_xor(sy, s);
    sx += __shfl_xor(sx, s);
  }
  if (lane == 0) {
    red[wave][0] = sy;
    red[wave][1] = sx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float* bo = p.bpart + (size_t)p.Cout * p.N;
    bo[((size_t)oy * p.N + n) * bpp + blk] = ((red[0][0] + red[1][0]) + red[2][0]) + red[3][0];
    bo[((size_t)(oy + 1) * p.N + n) * bpp + blk] = ((red[0][1] + red[1][1]) + red[2][1]) + red[3][1];
  }
}


// ---------------------------------------------------------------------------
// dW_off partials.  GEMM rows o (MB blocks of 32 starting at o0), columns
// (tap, channel) for a 32-channel slice, depth = output pixels of one row at a
// time.  Per output row the KH input rows it reads are staged channel-major
// in LDS ([c][i][column], zero outside the image) with the dOffset rows
// ([o][pixel], dtype); wave w owns taps tg+w, tg+w+4, tg+w+8.
struct WoffParams {
  int N, Cin, H, W, Ho, Wo, KH, KW, SH, SW, PH, PW, DH, DW, K2, Oc;
  int o0, orows, slices, bands, band_rows, num_wg, WoP, XR, XS, XL, DLS;
  const void* x;
  const float* doff;
  const bf16_t* doff16;  // dOffset rounded to bf16, or null
  float* part;  // [N*bands][Oc][K2][Cin]
  const bf16_t* xh;  // channel-minor copy of x left by a direct-gather forward, or null
};

// dW_off partial of one (image, 32-channel slice, band of output rows): a
// GEMM with rows = offset channels, columns = (tap, channel), depth = the
// band's output pixels.  The band's input rows are staged once (bf16:
// [row][pixel][32 channels]; fp32: [ch][row][XS], column XL is x = 0) and
// the taps read their shifted windows from LDS.  bf16 reads the dOffset
// operand straight from global memory as MFMA fragments (8 pixels of one
// offset channel per lane, rounded to bf16), one k-chunk ahead, in two fixed
// register slots; fp32 stages the dOffset rows too ([o][row][DLS]).
// A16: the dOffset operand comes from its bf16 copy in aligned 8-pixel
// pieces (bf16, one 32-row block, row length a multiple of 8): no fp32
// loads, registers for four waves per SIMD.
template <typename T, int MB, bool A16 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(A16 ? 4 : (MB == 1 ? 2 : 1)))) void k_woff_bwd(
    const WoffParams p) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int KC = 2 * VEC;  // pixels per k-chunk
  extern __shared__ __align__(16) unsigned char smem[];
  T* xs = (T*)smem;  // bf16: [XR][XS][32]; fp32: [32][XR][XS]
  T* dl = (T*)(smem + ((32 * p.XR * p.XS * (int)sizeof(T) + 15) & ~15));           // [MB*32][band_rows][DLS]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lw = xcd_swizzle(blockIdx.x, p.num_wg);
  const int per_img = p.slices * p.bands;
  const int n = lw / per_img, r = lw - n * per_img;
  const int band = r / p.slices, cs = r - band * p.slices;
  const int ho0 = band * p.band_rows, nrows = min(p.Ho, ho0 + p.band_rows) - ho0;
  const int HoWo = p.Ho * p.Wo;
  const int cl = lane & 31, half = lane >> 5;
  const int c = cs * 32 + cl;
  const T* __restrict__ x = (const T*)p.x;
  const float* __restrict__ doff = p.doff + (size_t)n * p.Oc * HoWo;
  const int y0 = ho0 * p.SH - p.PH;  // first input row of the band
  // ---- stage the band's input rows and dOffset rows ----
  // bf16: x as [row][pixel][32 channels] (pixel = x + PW), read as MFMA
  // fragments with transposed LDS reads; fp32: [channel][row][XS].
  constexpr bool kHwc = sizeof(T) == 2;
  if constexpr (kHwc) {
    const int nc = min(32, p.Cin - cs * 32);
    if (p.xh) {
      // from the channel-minor copy: buffer-to-LDS loads of 16-byte pieces
      // (4 per staged pixel), awaited after the dOffset rows are staged
      const int HWi = p.H * p.W;
      const rsrc_t xr = make_rsrc(p.xh + (size_t)n * (HWi + 1) * p.Cin, (uint32_t)((size_t)(HWi + 1) * p.Cin * 2));
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const int nslots = p.XR * p.XS * 4;
      for (int s0 = wv * 64; s0 < nslots; s0 += 256) {
        const int sl = s0 + lane, px = sl >> 2, pc = sl & 3;
        const int ry = px / p.XS, rx = px - ry * p.XS;
        const int y = y0 + ry, xx = rx - p.PW;
        const int pix = ((unsigned)y < (unsigned)p.H && (unsigned)xx < (unsigned)p.W) ? y * p.W + xx : HWi;
        const int voff = pc * 8 < nc ? (pix * p.Cin + cs * 32 + pc * 8) * 2 : kOOB;
        if (sl < nslots) load_lds16(xr, (unsigned char*)xs + s0 * 16, voff);  // lanes past the region write nothing
      }
    } else {
      const FastDiv drh = make_fastdiv(p.XR);
      const StageGeom sg = stage_geom<T>(p.W, -p.PW, p.XS, (size_t)p.Cin * p.H * p.W);
      stage_region<T>(xs, x, p.Cin, p.H, p.W, n, cs * 32, nc, y0, -p.PW, p.XR, p.XS, drh, sg, 32);
    }
  } else {
    const int tot = 32 * p.XR * p.XS;
    for (int e = tid; e < tot; e += 256) {
      const int cc = e / (p.XR * p.XS), rr = e - cc * (p.XR * p.XS);
      const int ry = rr / p.XS, xi = rr - ry * p.XS;
      const int y = y0 + ry, xx = xi - p.XL;
      const int ch = cs * 32 + cc;
      T v = zero_elem<T>();
      if (ch < p.Cin && (unsigned)y < (unsigned)p.H && (unsigned)xx < (unsigned)p.W)
        v = x[(((size_t)n * p.Cin + ch) * p.H + y) * p.W + xx];
      xs[e] = v;
    }
  }
  if constexpr (kHwc) {
    // the dOffset operand is read in the tap loop below
  } else if (sizeof(T) == 2 && (p.Wo & 3) == 0 && (HoWo & 3) == 0 && (p.DLS & 3) == 0) {
    // four pixels per piece (one 16-byte load, one 8-byte store), eight
    // pieces per thread per pass; padding rows and columns are zero
    const int pr = p.DLS >> 2, rowp = p.band_rows * pr;
    const int tot = MB * 32 * rowp;
    const FastDiv drow = make_fastdiv(rowp), dpr = make_fastdiv(pr);
    for (int e0 = tid; e0 < tot; e0 += 256 * 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * 256;
        const int o = fdiv(e, drow), rr = e - o * rowp;
        const int ry = fdiv(rr, dpr), w4 = (rr - ry * pr) * 4;
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e < tot && o < p.orows && ry < nrows && w4 < p.Wo)
          v[u] = *(const float4*)(doff + (size_t)(p.o0 + o) * HoWo + (size_t)(ho0 + ry) * p.Wo + w4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (e0 + u * 256 < tot)
          *(uint2*)(dl + (e0 + u * 256) * 4) = make_uint2(pack_bf16x2(v[u].x, v[u].y), pack_bf16x2(v[u].z, v[u].w));
    }
  } else {
    // eight elements per thread per pass, all loads of a pass in flight
    const int rowlen = p.band_rows * p.DLS;
    const int tot = MB * 32 * rowlen;
    const FastDiv drow = make_fastdiv(rowlen), dls = make_fastdiv(p.DLS);
    for (int e0 = tid; e0 < tot; e0 += 256 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * 256;
        const int o = fdiv(e, drow), rr = e - o * rowlen;
        const int ry = fdiv(rr, dls), wo = rr - ry * p.DLS;
        v[u] = 0.f;
        if (e < tot && o < p.orows && ry < nrows && wo < p.Wo)
          v[u] = doff[(size_t)(p.o0 + o) * HoWo + (size_t)(ho0 + ry) * p.Wo + wo];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (e0 + u * 256 < tot) dl[e0 + u * 256] = Elem<T>::from_f32(v[u]);
    }
  }
  if (kHwc && p.xh) wait_vm<0>();
  __syncthreads();
  if constexpr (kHwc) {
    // ---- taps in groups of 12 (three per wave) ----
    const int g4 = lane >> 4, j4 = lane & 15;
    // this lane's transposed-read position inside a tap's window
    const int lofs = 16 * (g4 & 1) + 4 * (j4 & 3) + (8 * (g4 >> 1) + (j4 >> 2)) * p.SW * 32;
    const int nkc = p.WoP / KC, niter = nrows * nkc;
    const FastDiv dk = make_fastdiv(nkc);
    const bool vec4 = (p.Wo & 3) == 0;
    // dOffset planes of this image through a buffer: loads of lanes with
    // nothing to load go past its range and read zero, so every step issues
    // the same loads and the waits for them stay exact
    const __amdgpu_buffer_rsrc_t drs = make_brsrc(doff, (uint32_t)((size_t)p.Oc * HoWo * 4));
    // the bf16 copy, where every 8-pixel group of a row is one aligned piece
    const __amdgpu_buffer_rsrc_t d16 =
        make_brsrc(A16 ? p.doff16 + (size_t)n * p.Oc * HoWo : nullptr, A16 ? (uint32_t)((size_t)p.Oc * HoWo * 2) : 0u);
    int orow[MB];  // element offset of this lane's offset channel (o0 + mb*32 + lane%32) at the band's first row
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int o = mb * 32 + cl;
      orow[mb] = o < p.orows ? (p.o0 + o) * HoWo + ho0 * p.Wo : -1;
    }
    // operand of k-chunk `it` (row it / nkc, pixels kc + 8*half .. +7)
    auto load_a = [&](int it, uint4* a) {
      const int ry = fdiv(it, dk), kc = (it - ry * nkc) * KC;
      const int w0 = kc + half * VEC;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bool ok = orow[mb] >= 0 && it < niter;
        const int e0 = orow[mb] + ry * p.Wo + w0;
        if constexpr (A16) {
          a[mb] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(d16, ok && w0 < p.Wo ? e0 * 2 : kOOB,
                                                                                 0, 0));
          continue;
        }
        const int b0 = e0 * 4;
        float f[8];
        if (vec4) {
          const uint4 u0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         drs, ok && w0 < p.Wo ? b0 : kOOB, 0, 0));
          const uint4 u1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         drs, ok && w0 + 4 < p.Wo ? b0 + 16 : kOOB, 0, 0));
          f[0] = __uint_as_float(u0.x); f[1] = __uint_as_float(u0.y);
          f[2] = __uint_as_float(u0.z); f[3] = __uint_as_float(u0.w);
          f[4] = __uint_as_float(u1.x); f[5] = __uint_as_float(u1.y);
          f[6] = __uint_as_float(u1.z); f[7] = __uint_as_float(u1.w);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            f[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(drs, ok && w0 + i < p.Wo ? b0 + 4 * i : kOOB,
                                                                        0, 0));
        }
        a[mb] = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                           pack_bf16x2(f[6], f[7]));
      }
    };
    for (int tg = 0; tg < p.K2; tg += 12) {
      f32x16_t acc[MB][3];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[mb][j][q] = 0.f;
      const T* tb[3];
      int ntap = 0;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int t = tg + wave + 4 * j;
        tb[j] = xs;
        if (t < p.K2) {
          const int ti = t / p.KW, tj = t - ti * p.KW;
          tb[j] = xs + ((size_t)ti * p.DH * p.XS + tj * p.DW) * 32 + lofs;
          ntap = j + 1;
        }
      }
      auto step = [&](int it, const uint4* a) {
        const int ry = fdiv(it, dk), kc = (it - ry * nkc) * KC;
        const int ofs = (ry * p.SH * p.XS + kc * p.SW) * 32;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          if (j >= ntap) break;
          uint2 hh[2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            hh[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                  (__attribute__((address_space(3))) bf16x4_t*)(
                                                      (const bf16_t*)tb[j] + ofs + h * 4 * p.SW * 32)));
          const uint4 b = make_uint4(hh[0].x, hh[0].y, hh[1].x, hh[1].y);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) mfma_chunk(acc[mb][j], a[mb], b, T());
        }
      };
      // four fixed slots, each operand loaded three k-chunks before its use
      uint4 a0[MB], a1[MB], a2[MB], a3[MB];
      load_a(0, a0);
      load_a(1, a1);
      load_a(2, a2);
      for (int it = 0; it < niter; it += 4) {
        load_a(it + 3, a3);
        step(it, a0);
        load_a(it + 4, a0);
        if (it + 1 < niter) step(it + 1, a1);
        load_a(it + 5, a1);
        if (it + 2 < niter) step(it + 2, a2);
        load_a(it + 6, a2);
        if (it + 3 < niter) step(it + 3, a3);
      }
      float* part = p.part + (size_t)(n * p.bands + band) * p.Oc * p.K2 * p.Cin;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int t = tg + wave + 4 * j;
        if (t >= p.K2) break;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            const int o = mb * 32 + acc_row(lane, q);
            if (o < p.orows && c < p.Cin) part[((size_t)(p.o0 + o) * p.K2 + t) * p.Cin + c] = acc[mb][j][q];
          }
      }
    }
    return;
  }
  // ---- taps in groups of 12 (three per wave) ----
  for (int tg = 0; tg < p.K2; tg += 12) {
    f32x16_t acc[MB][3];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[mb][j][q] = 0.f;
    for (int ry = 0; ry < nrows; ++ry) {
      for (int kc = 0; kc < p.WoP; kc += KC) {
        const int w0 = kc + half * VEC;
        uint4 a[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) a[mb] = *(const uint4*)(dl + ((mb * 32 + cl) * p.band_rows + ry) * p.DLS + w0);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const int t = tg + wave + 4 * j;
          if (t >= p.K2) break;
          const int ti = t / p.KW, tj = t - ti * p.KW;
          uint4 b;
          if constexpr (kHwc) {
            // lane: channel n = lane % 32, pixels kc + 8*(lane/32) + 0..7, as
            // two transposed reads of 4 pixel rows x 4 channels per 16 lanes
            const int g4 = lane >> 4, j4 = lane & 15;
            const T* rowb = xs + (size_t)(ry * p.SH + ti * p.DH) * p.XS * 32 + 16 * (g4 & 1) + 4 * (j4 & 3);
            uint2 hh[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int wo = kc + 8 * (g4 >> 1) + 4 * h + (j4 >> 2);
              const bf16_t* a16 = (const bf16_t*)(rowb + (size_t)(wo * p.SW + tj * p.DW) * 32);
              typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
              hh[h] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                    (__attribute__((address_space(3))) bf16x4_t*)a16));
            }
            b = make_uint4(hh[0].x, hh[0].y, hh[1].x, hh[1].y);
          } else {
            const T* src = xs + (cl * p.XR + ry * p.SH + ti * p.DH) * p.XS + p.XL - p.PW + tj * p.DW + w0 * p.SW;
            T v[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = src[e * p.SW];
            b = *(const uint4*)v;
          }
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) mfma_chunk(acc[mb][j], a[mb], b, T());
        }
      }
    }
    float* part = p.part + (size_t)(n * p.bands + band) * p.Oc * p.K2 * p.Cin;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int t = tg + wave + 4 * j;
      if (t >= p.K2) break;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int o = mb * 32 + acc_row(lane, q);
          if (o < p.orows && c < p.Cin) part[((size_t)(p.o0 + o) * p.K2 + t) * p.Cin + c] = acc[mb][j][q];
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Final dX: dx[n][c][y][x] = dtype(dX_offset + the sampling part of dX).
// dX_offset is a GEMM with rows = 64 input pixels, columns c (one 32-channel
// block per wave), depth kk = o*K2 + tap (padded to KKP, in chunks of KKC);
// its pixel operand [pixel][kk] (dOffset at the output pixel whose tap lands
// on the input pixel, or 0) is built in LDS.  With pixels as rows, a lane's
// accumulators hold one channel, and the lanes of a row 32 consecutive
// channels: the channel-minor sampling part is read in 128-byte runs.
struct DxParams {
  int N, Cin, H, W, Ho, Wo, KH, KW, SH, SW, PH, PW, DH, DW, K2, Oc, KKP, KKC;
  int pix_blocks, cblocks, num_wg;
  FastDiv div_w, div_sh, div_sw;
  const void* wofft;  // [Cin][KKP]
  const float* doff;
  const float* dxs;   // sampling part of dX, fp32, channel-minor [N][H][W][Cin]
  void* dx;
};

template <typename T>
__global__ __launch_bounds__(512) void k_dx_final(const DxParams p) {
  constexpr int VEC = Elem<T>::VEC;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lw = xcd_swizzle(blockIdx.x, p.num_wg);
  const int per_img = p.pix_blocks * p.cblocks;
  const int n = lw / per_img, r = lw - n * per_img;
  const int pbk = r / p.cblocks, cb = r - pbk * p.cblocks;
  const int HW = p.H * p.W, HoWo = p.Ho * p.Wo;
  const int pix0 = pbk * 64;
  const int bstr = p.KKC + VEC;
  T* bt = (T*)smem;  // [64][bstr]
  const float* __restrict__ doff = p.doff + (size_t)n * p.Oc * HoWo;
  const int c0 = cb * 256 + wave * 32;  // eight waves, 32 channels each
  const bool active = c0 < p.Cin;
  const T* __restrict__ wt = (const T*)p.wofft;
  const __amdgpu_buffer_rsrc_t wrs = make_brsrc(wt, (uint32_t)((size_t)p.Cin * p.KKP * sizeof(T)));
  f32x16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.f;
  const int crow = c0 + (lane & 31);
  // The sampling part of dX at this lane's accumulator elements (channel
  // crow; pixels pix0 + j*32 + acc_row(lane, r)), loaded up front so the
  // loads overlap the dOffset tile and the MFMAs, and added after them.
  float sv[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int q = pix0 + j * 32 + acc_row(lane, r);
      sv[j][r] = active && crow < p.Cin && q < HW ? p.dxs[((size_t)n * HW + q) * p.Cin + crow] : 0.f;
    }
  int4* kinfo = (int4*)(smem + ((64 * bstr * (int)sizeof(T) + 15) & ~15));  // [KKC]
  for (int kb = 0; kb < p.KKP; kb += p.KKC) {
    const int len = min(p.KKC, p.KKP - kb);
    __syncthreads();
    // per depth index kk = o*K2 + tap: dOffset plane and the tap's shift
    for (int kl = tid; kl < len; kl += 512) {
      const int kk = kb + kl;
      int4 ki = make_int4(-1, 0, 0, 0);
      if (kk < p.Oc * p.K2) {
        const int o = kk / p.K2, t = kk - o * p.K2;
        const int ti = t / p.KW, tj = t - ti * p.KW;
        ki = make_int4(o * HoWo, p.PH - ti * p.DH, p.PW - tj * p.DW, 0);
      }
      kinfo[kl] = ki;
    }
    __syncthreads();
    // B tile: dOffset at the output pixel whose tap lands on the input pixel.
    // Lane = pixel, wave = a run of eight consecutive depth indices (runs
    // stepping by 64; len is a multiple of 16): each of a wave's gathers
    // reads one dOffset plane at a shifted run of consecutive pixels, a few
    // cache lines, eight per thread in flight at a time; the run goes to LDS
    // in 16-byte writes (rows 16-byte aligned, no bank conflicts)
    {
      const int pix = tid & 63;
      const int q = pix0 + pix;
      const int y = fdiv(q, p.div_w), xx = q - y * p.W;
      for (int k0 = wave * 8; k0 < len; k0 += 8 * 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kl = k0 + u;
          const int4 ki = kinfo[kl];
          v[u] = 0.f;
          const int ny = y + ki.y, nx = xx + ki.z;
          if (ki.x >= 0 && q < HW && ny >= 0 && nx >= 0) {
            int ho = ny, wo = nx;
            bool ok = true;
            if (p.SH != 1) { ho = fdiv(ny, p.div_sh); ok = ho * p.SH == ny; }
            if (p.SW != 1) { wo = fdiv(nx, p.div_sw); ok = ok && wo * p.SW == nx; }
            if (ok && ho < p.Ho && wo < p.Wo) v[u] = doff[(size_t)ki.x + (size_t)ho * p.Wo + wo];
          }
        }
        alignas(16) T o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) o[u] = Elem<T>::from_f32(v[u]);
        uint4* dst = (uint4*)(bt + pix * bstr + k0);
#pragma unroll
        for (int h = 0; h < (int)sizeof(o) / 16; ++h) dst[h] = ((const uint4*)o)[h];
      }
    }
    __syncthreads();
    if (active) {
      // The weight operand of k-chunk kc comes from global memory three
      // chunks ahead, in three fixed register slots (the loop is unrolled by
      // three); the loads are always issued (past the chunks or the channels
      // they read zero), so the compiler's waits stay exact.
      const int nkc = len / (2 * VEC);
      auto lda = [&](int kc) {
        const int kl = kc * 2 * VEC + (lane >> 5) * VEC;
        const int off = kc < nkc && crow < p.Cin ? (crow * p.KKP + kb + kl) * (int)sizeof(T) : kOOB;
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, 0));
      };
      auto mm = [&](int kc, const uint4& a) {
        if (kc >= nkc) return;
        const int kl = kc * 2 * VEC + (lane >> 5) * VEC;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4 b = *(const uint4*)(bt + (j * 32 + (lane & 31)) * bstr + kl);
          mfma_chunk(acc[j], b, a, T());  // rows = pixels, columns = channels
        }
      };
      uint4 a0 = lda(0), a1 = lda(1), a2 = lda(2);
      for (int kc = 0; kc < nkc; kc += 3) {
        mm(kc, a0);
        a0 = lda(kc + 3);
        mm(kc + 1, a1);
        a1 = lda(kc + 4);
        mm(kc + 2, a2);
        a2 = lda(kc + 5);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] += sv[j][r];
  T* dx = (T*)p.dx;
  // whole 8-pixel pieces need HW % 8 == 0 (a piece never straddles a plane)
  if ((HW & 7) == 0) {
    // through LDS: each wave's 32 channels x 64 pixels (fp32, rows padded
    // to 68 floats), then per lane 8 consecutive pixels of one channel: one
    // 32-byte read, one 16-byte (bf16) store
    __syncthreads();  // the B tile is no longer read
    float* ep = (float*)smem + wave * 32 * 68;
    if (active) {
      // four consecutive pixels of the lane's channel per 16-byte write
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(float4*)(ep + (lane & 31) * 68 + j * 32 + acc_row(lane, 4 * r4)) =
              make_float4(acc[j][4 * r4], acc[j][4 * r4 + 1], acc[j][4 * r4 + 2], acc[j][4 * r4 + 3]);
    }
    // a wave reads back only its own block: its LDS operations execute in
    // issue order, so only the compiler has to be kept from reordering
    asm volatile("" ::: "memory");
    if (!active) return;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int cl = k * 8 + (lane >> 3), ql = (lane & 7) * 8, q = pix0 + ql, cc = c0 + cl;
      if (q >= HW || cc >= p.Cin) continue;
      const float4 a0 = *(const float4*)(ep + cl * 68 + ql), a1 = *(const float4*)(ep + cl * 68 + ql + 4);
      float f[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      store8(dx + ((size_t)n * p.Cin + cc) * HW + q, f);
    }
    return;
  }
  if (!active) return;
  if (crow >= p.Cin) return;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r2 = 0; r2 < 16; ++r2) {
      const int q = pix0 + j * 32 + acc_row(lane, r2);
      if (q < HW) dx[((size_t)n * p.Cin + crow) * HW + q] = Elem<T>::from_f32(acc[j][r2]);
    }
}

// ---------------------------------------------------------------------------
// Prep: W2[(t,c)][co] = W[co][c][t]; WoffT[c][o*K2+t] = W_off[o][c][t] (zero
// for kk >= Oc*K2); the nz0 floats at z0 zeroed.
template <typename T>
__device__ __forceinline__ void prep_backward_body(int bid, int nblocks, const T* __restrict__ w,
                                                   const T* __restrict__ w_off, T* w2, T* wofft, float* z0,
                                                   size_t nz0, int Cout, int Cin, int K2, int Oc, int KKP) {
  const size_t n1 = (size_t)Cout * K2 * Cin, n2 = (size_t)Cin * KKP;
  const size_t nz4 = nz0 / 4;
  const size_t total = n1 + n2 + nz4 + (nz0 & 3);
  for (size_t e = (size_t)bid * 256 + threadIdx.x; e < total; e += (size_t)nblocks * 256) {
    // weight tensors are far below 2^31 elements: 32-bit index arithmetic
    if (e < n1) {
      const int ei = (int)e;
      const int r = ei / Cout, co = ei - r * Cout;
      const int t = r / Cin, c = r - t * Cin;
      w2[e] = w[(co * Cin + c) * K2 + t];
    } else if (e < n1 + n2) {
      const int f = (int)(e - n1);
      const int c = f / KKP, kk = f - c * KKP;
      const int o = kk / K2;
      wofft[f] = kk < Oc * K2 ? w_off[(o * Cin + c) * K2 + (kk - o * K2)] : zero_elem<T>();
    } else if (e < n1 + n2 + nz4) {
      ((float4*)z0)[e - n1 - n2] = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      z0[nz4 * 4 + (e - n1 - n2 - nz4)] = 0.f;
    }
  }
}

// Sum of dY over the pixels of one (output channel, image) plane, by one
// wave: the bias partial part[ch * N + n].  bf16 planes whose length allows
// it are read as 16-byte pieces, four per lane in flight; the lanes' sums are
// then added in a fixed order.
template <typename T>
__device__ __forceinline__ void bias_dy_body(const T* __restrict__ dy, float* part, int Cout, int N, int HoWo, int ch,
                                             int n) {
  const int lane = threadIdx.x & 63;
  const size_t base = ((size_t)n * Cout + ch) * HoWo;
  float s = 0.f;
  if (sizeof(T) == 2 && (HoWo & 7) == 0) {
    const uint4* src = (const uint4*)((const bf16_t*)dy + base);
    const int nv = HoWo >> 3;
    for (int q0 = lane; q0 < nv; q0 += 4 * 64) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = q0 + u * 64 < nv ? src[q0 + u * 64] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float f[8];
        unpack8(v[u], f);
        s += ((f[0] + f[1]) + (f[2] + f[3])) + ((f[4] + f[5]) + (f[6] + f[7]));
      }
    }
  } else {
    for (int q = lane; q < HoWo; q += 64) s += Elem<T>::to_f32(dy[base + q]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) part[(size_t)ch * N + n] = s;
}

// The backward's preparation in one launch: workgroups [0, num_tg) build the
// candidate lists, the next ceil(Cout*N / 4) sum dY per (channel, image)
// plane, one wave per plane, the rest lay out W2 and W_off^T and zero the
// dOffset partials and the max word.
template <typename T>
__global__ __launch_bounds__(256) void k_prep_backward(const BwdParams b, const T* __restrict__ w,
                                                       const T* __restrict__ w_off, T* w2, T* wofft, float* z0,
                                                       size_t nz0, int Cout, int Cin, int K2, int Oc, int KKP,
                                                       const T* __restrict__ dy, float* bpart, int N, int HoWo) {
  const int bid = (int)blockIdx.x;
  const int nbias = (Cout * N + 3) / 4;
  if (bid < b.num_tg) {
    bwd_lists_body(b, bid);
  } else if (bid < b.num_tg + nbias) {
    const int r = (bid - b.num_tg) * 4 + (int)(threadIdx.x >> 6);
    if (r < Cout * N) bias_dy_body<T>(dy, bpart, Cout, N, HoWo, r % Cout, r / Cout);
  } else {
    const int base = b.num_tg + nbias;
    prep_backward_body<T>(bid - base, (int)gridDim.x - base, w, w_off, w2, wofft, z0, nz0, Cout, Cin, K2, Oc, KKP);
  }
}

// All weight and bias gradients from their partials, summed in a fixed order
// and rounded once: dw[co][c][t] (from [ndw][co][t][c], one partial per
// pixel range of the dW GEMM), dw_off[o][c][t] (from
// [N*bands][o][t][c]), db (from [co][N]), db_off (from [o][N][blocks of 256
// pixels]).  The first workgroups take the bias channels, one wave each (its
// lanes add strided partials in ascending order, then a fixed xor tree).
// Every other thread sums one weight element's partials in ascending order
// with up to 32 loads in flight; the dw_off elements, which have the most
// partials (one per image and band), come first so that they are not left for
// the end of the launch.
template <typename T>
__global__ __launch_bounds__(256) void k_reduce_final(const float* __restrict__ dwpart, int ndw, T* dw, int Cout,
                                                      const float* __restrict__ dwoffpart, T* dwoff, int Oc, int nwp,
                                                      const float* __restrict__ bpart, T* db, T* dboff, int N, int Cin,
                                                      int K2, int nbo) {
  const int nch = Cout + Oc;
  const int nbw = (nch + 3) / 4;  // the first workgroups: one wave per bias channel
  if ((int)blockIdx.x < nbw) {
    const int ch = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (ch >= nch) return;
    T* dst = ch < Cout ? db : dboff;
    if (!dst) return;
    const float* src = ch < Cout ? bpart + (size_t)ch * N : bpart + (size_t)Cout * N + (size_t)(ch - Cout) * nbo;
    const int cnt = ch < Cout ? N : nbo;
    float s = 0.f;
    for (int z = lane; z < cnt; z += 64) s += src[z];  // each lane in ascending order, then a fixed tree
    for (int k = 32; k > 0; k >>= 1) s += __shfl_xor(s, k);
    if (lane == 0) dst[ch < Cout ? ch : ch - Cout] = Elem<T>::from_f32(s);
    return;
  }
  const size_t ck = (size_t)Cin * K2;
  const size_t n1 = (size_t)Cout * ck, n2 = (size_t)Oc * ck;
  const size_t b0 = blockIdx.x - nbw, nb = gridDim.x - nbw;
  for (size_t e = b0 * 256 + threadIdx.x; e < n1 + n2; e += nb * 256) {
    const bool woff = e < n2;
    const size_t f = woff ? e : e - n2;  // partial order: [o][t][c]
    const int fi = (int)f;               // weight tensors: below 2^31 elements
    const int r = fi / Cin, c = fi - r * Cin;
    const int o = r / K2, t = r - o * K2;
    const float* src = woff ? dwoffpart : dwpart;
    const size_t stride = woff ? n2 : n1;
    const int cnt = woff ? nwp : ndw;
    float s = 0.f;
    for (int z = 0; z < cnt; z += 32) {
      float v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = z + u < cnt ? src[(size_t)(z + u) * stride + f] : 0.f;
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (z + u < cnt) s += v[u];
    }
    (woff ? dwoff : dw)[((size_t)o * Cin + c) * K2 + t] = Elem<T>::from_f32(s);
  }
}

// ---------------------------------------------------------------------------
static unsigned grid_cap(size_t total, unsigned cap) {
  size_t g = (total + 255) / 256;
  if (g > cap) g = cap;
  return (unsigned)(g ? g : 1);
}

template <typename T>
static hipError_t backward_t(const deft_plan& p, const BackwardArgs& a, hipStream_t st) {
  const deft_desc& d = p.d;
  char* ws = a.ws;
  T* w2 = (T*)(ws + p.ws_w2);
  T* wofft = (T*)(ws + p.ws_wofft);
  T* dcol = (T*)(ws + p.ws_dcol);
  const T* cols = (const T*)(ws + p.ws_cols);
  float* dxs = (float*)(ws + p.ws_dx32);
  float* doff = (float*)(ws + p.ws_doff);
  float* doffp = (float*)(ws + p.ws_doffp);
  uint32_t* maxbits = (uint32_t*)(ws + p.ws_maxbits);
  int4* lists = (int4*)(ws + p.ws_list);
  float* dwpart = (float*)(ws + p.ws_dwpart);
  float* dwoffpart = (float*)(ws + p.ws_dwoffpart);
  float* bpart = (float*)(ws + p.ws_biaspart);
  hipError_t e;
  BwdParams b;
  b.N = d.n; b.Cin = d.c_in; b.H = d.h; b.W = d.w; b.Ho = p.ho; b.Wo = p.wo; b.KH = d.kh; b.KW = d.kw;
  b.SH = d.stride_h; b.SW = d.stride_w; b.PH = d.pad_h; b.PW = d.pad_w; b.DH = d.dil_h; b.DW = d.dil_w;
  b.G = d.offset_groups; b.Cg = p.cg; b.K2 = p.taps; b.Oc = p.oc; b.Ck = p.ck;
  b.CH = p.btile_h; b.CW = p.btile_w; b.bt_h = p.btiles_h; b.bt_w = p.btiles_w; b.halo = p.bhalo;
  b.CC = p.chunk_b;
  b.dcstr = p.chunk_b + (p.bwd_mf ? 16 : (d.dtype == DEFT_BF16 ? 8 : 4));
  b.num_wg = p.num_btiles * d.offset_groups * (p.cg / p.chunk_b); b.list_cap = p.list_cap + 64;  // list stride: room for the last block's filler entries
  int cb = 0;
  while ((1 << cb) < p.list_cap + 1) ++cb;
  b.capbits = cb;
  b.xstr = p.bwd_mf ? p.chunk_b : p.chunk_b + (d.dtype == DEFT_BF16 ? 8 : 4);
  b.lds_dx = p.lb_dx; b.lds_dc = p.lb_dc; b.lds_cnt = p.lb_cnt;
  b.x = a.x; b.off = a.offsets; b.dcol = dcol; b.maxbits = maxbits; b.dxs = dxs; b.doffp = doffp;
  b.lists = lists;
  b.doff = doff; b.bpart = bpart; b.Cout = d.c_out;
  b.doff16 = d.dtype == DEFT_BF16 ? (bf16_t*)(ws + p.ws_doff16) : nullptr;
  b.xh = (p.direct && p.bwd_mf) ? (const bf16_t*)(ws + p.ws_xh) : nullptr;
  b.num_tg = p.num_btiles * d.offset_groups;
  b.counts = (int*)(ws + p.ws_lcount);
  {
    // candidate lists, dY bias sums, W2 / W_off^T, and zero the max |dCol|
    // word (the dOffset partials are all written by the two sampling kernels)
    const size_t nz = 4;
    const size_t total = (size_t)d.c_out * p.ck + (size_t)d.c_in * p.kk_pad + nz / 4 + 4;
    const unsigned grid = (unsigned)b.num_tg + (unsigned)((d.c_out * d.n + 3) / 4) + grid_cap(total, 512);
    DEFT_LAUNCH("prep_backward", k_prep_backward<T>, dim3(grid), dim3(256), 0, st, b, (const T*)a.w,
                (const T*)a.w_off, w2, wofft, (float*)maxbits, nz, d.c_out, d.c_in, p.taps, p.oc, p.kk_pad, (const T*)a.dy,
                bpart, d.n, p.ho * p.wo);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = launch_gemm_dcol(p, w2, a.dy, dcol, p.bwd_mf ? nullptr : maxbits, st);  // the MFMA scatter needs no max
  if (e != hipSuccess) return e;
  e = launch_gemm_dw(p, a.dy, cols, dwpart, st);
  if (e != hipSuccess) return e;

  // sampling backward, then dOffset of every pair (with the taps beyond the halo)
  {
    auto kern = !p.bwd_mf ? k_sample_bwd<T> : p.chunk_b == 64 ? k_sample_bwd_mf<64> : k_sample_bwd_mf<32>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, p.lb_total);
    if (e != hipSuccess) return e;
    if (b.num_wg) DEFT_LAUNCH("sample_backward", kern, dim3(b.num_wg), dim3(256), p.lb_total, st, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one workgroup per 256 pixels of each (image, group, tap) plane
    const size_t mgrid = (size_t)d.n * d.offset_groups * p.taps * (size_t)((p.ho * p.wo + 255) / 256);
    if (mgrid > 0x7fffffffu) return hipErrorInvalidValue;
    if (mgrid) DEFT_LAUNCH("sample_backward_miss", k_sample_bwd_miss<T>, dim3((unsigned)mgrid), dim3(256), 0, st, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // offset-conv weight gradient partials
  {
    WoffParams w;
    w.N = d.n; w.Cin = d.c_in; w.H = d.h; w.W = d.w; w.Ho = p.ho; w.Wo = p.wo; w.KH = d.kh; w.KW = d.kw;
    w.SH = d.stride_h; w.SW = d.stride_w; w.PH = d.pad_h; w.PW = d.pad_w; w.DH = d.dil_h; w.DW = d.dil_w;
    w.K2 = p.taps; w.Oc = p.oc;
    w.slices = (d.c_in + 31) / 32;
    w.bands = p.woff_bands;
    w.band_rows = (p.ho + w.bands - 1) / w.bands;
    w.num_wg = d.n * w.slices * w.bands;
    const int kc = d.dtype == DEFT_BF16 ? 16 : 8;
    w.WoP = (p.wo + kc - 1) / kc * kc;
    w.XR = (w.band_rows - 1) * d.stride_h + (d.kh - 1) * d.dil_h + 1;
    // staged row: columns [-XL, XS - XL) of x, XL = pad_w (the fp32 path's
    // column of x = 0; the bf16 path indexes pixels from x = -PW directly)
    const int span = (w.WoP - 1) * d.stride_w + (d.kw - 1) * d.dil_w + 1;  // from x = -PW
    w.XL = d.pad_w;
    w.XS = span;  // pixels per staged row, from x = -PW
    w.DLS = w.WoP + (d.dtype == DEFT_BF16 ? 8 : 4);
    w.x = a.x; w.doff = doff; w.part = dwoffpart;
    w.doff16 = b.doff16;
    w.xh = p.direct ? (const bf16_t*)(ws + p.ws_xh) : nullptr;
    for (int o0 = 0; o0 < p.oc && w.num_wg; o0 += 96) {
      w.o0 = o0;
      w.orows = p.oc - o0 < 96 ? p.oc - o0 : 96;
      const int mb = (w.orows + 31) / 32;
      const int lds = ((32 * w.XR * w.XS * (int)sizeof(T) + 15) & ~15) +
                      (sizeof(T) == 2 ? 0 : mb * 32 * w.band_rows * w.DLS * (int)sizeof(T));
      if (mb == 1 && woff_a16(d.dtype, p.oc, p.wo)) {
        e = hipFuncSetAttribute((const void*)k_woff_bwd<T, 1, true>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess)
          DEFT_LAUNCH("offset_weight_backward", (k_woff_bwd<T, 1, true>), dim3(w.num_wg), dim3(256), lds, st, w);
      } else if (mb == 1) {
        e = hipFuncSetAttribute((const void*)k_woff_bwd<T, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess)
          DEFT_LAUNCH("offset_weight_backward", (k_woff_bwd<T, 1>), dim3(w.num_wg), dim3(256), lds, st, w);
      } else if (mb == 2) {
        e = hipFuncSetAttribute((const void*)k_woff_bwd<T, 2>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess)
          DEFT_LAUNCH("offset_weight_backward", (k_woff_bwd<T, 2>), dim3(w.num_wg), dim3(256), lds, st, w);
      } else {
        e = hipFuncSetAttribute((const void*)k_woff_bwd<T, 3>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess)
          DEFT_LAUNCH("offset_weight_backward", (k_woff_bwd<T, 3>), dim3(w.num_wg), dim3(256), lds, st, w);
      }
      if (e != hipSuccess) return e;
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  // final dX
  {
    DxParams q;
    q.N = d.n; q.Cin = d.c_in; q.H = d.h; q.W = d.w; q.Ho = p.ho; q.Wo = p.wo; q.KH = d.kh; q.KW = d.kw;
    q.SH = d.stride_h; q.SW = d.stride_w; q.PH = d.pad_h; q.PW = d.pad_w; q.DH = d.dil_h; q.DW = d.dil_w;
    q.K2 = p.taps; q.Oc = p.oc; q.KKP = p.kk_pad;
    q.KKC = p.kk_pad < 256 ? p.kk_pad : 256;
    q.pix_blocks = (d.h * d.w + 63) / 64;
    q.cblocks = (d.c_in + 255) / 256;
    q.num_wg = d.n * q.pix_blocks * q.cblocks;
    q.wofft = wofft; q.doff = doff; q.dxs = dxs; q.dx = a.dx;
    q.div_w = make_fastdiv(d.w); q.div_sh = make_fastdiv(d.stride_h); q.div_sw = make_fastdiv(d.stride_w);
    const int lds = std::max(((64 * (q.KKC + (d.dtype == DEFT_BF16 ? 8 : 4)) * (int)sizeof(T) + 15) & ~15) + q.KKC * 16,
                             8 * 32 * 68 * 4);  // B tile + tap table, or the epilogue's fp32 blocks
    auto kern = k_dx_final<T>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    if (q.num_wg) DEFT_LAUNCH("dx_final", kern, dim3(q.num_wg), dim3(512), lds, st, q);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // bias partials, then every weight / bias gradient
  {
    const size_t total = ((size_t)d.c_out + p.oc) * p.ck;
    const unsigned nbw = (unsigned)(d.c_out + p.oc + 3) / 4;  // bias workgroups, then the weight sums
    DEFT_LAUNCH("reduce_final", k_reduce_final<T>, dim3(nbw + grid_cap(total, 4096)), dim3(256), 0, st, dwpart, p.dw_splits, (T*)a.dw,
                d.c_out, dwoffpart, (T*)a.dw_off, p.oc, d.n * p.woff_bands, bpart, (T*)a.db, (T*)a.db_off, d.n,
                d.c_in, p.taps, d.n * ((p.ho * p.wo + 255) / 256));
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_backward(const deft_plan& p, const BackwardArgs& a, hipStream_t st) {
  return p.d.dtype == DEFT_BF16 ? backward_t<bf16_t>(p, a, st) : backward_t<float>(p, a, st);
}

}  // namespace deft
