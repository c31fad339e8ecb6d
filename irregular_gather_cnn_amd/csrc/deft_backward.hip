// Backward pass of the deformable convolution layer for gfx950.
//
// The DefT explainer page speaks of training time only ("The argument in one
// glance", "This paper's idea"), so the backward is the exact derivative of
// the forward: dCol = W^T dY and dW = dY Col run on the MFMA GEMMs
// (deft_gemm.hip); this file holds
//   k_sample_bwd  -- per output tile: re-derives each tap's corner and weights
//                    from the saved offsets, scatters dCol times the bilinear
//                    weights into an LDS copy of the tile's halo region
//                    (fp32 LDS atomics) that is then added to dX with global
//                    atomics, and reduces dOffset = sum over the group's
//                    channels of dCol times the corner differences;
//   k_woff_bwd    -- dW_off = dOffset against the plain patches of x (MFMA,
//                    per image and channel slice) and db_off;
//   k_dx_off      -- dX_offset, the transposed offset convolution of dOffset
//                    (MFMA, per input tile), added to the accumulated dX and
//                    rounded once to the output dtype;
//   finalize / prep kernels (weight transposes, fp32 -> dtype, bias sums).
#include "deft_device.h"
#include "deft_internal.h"

namespace deft {

hipError_t launch_gemm_dcol(const deft_plan& p, const void* w2, const void* dy, void* dcol, hipStream_t st);
hipError_t launch_gemm_dw(const deft_plan& p, const void* dy, const void* cols, float* dw32, hipStream_t st);

struct BwdParams {
  int N, Cin, H, W, Ho, Wo, KH, KW, SH, SW, PH, PW, DH, DW, G, Cg, K2, Oc, Ck, Cout;
  int TH, TW, halo, CC, GW, gsplit, tiles_h, tiles_w, num_wg;
  int FH, FW, pstr, dstr, lognv;
  int lds_x, lds_dx, lds_off, lds_info, lds_doff;
  FastDiv div_tw, div_k2;
  const void* x;
  const float* off;
  const void* dcol;
  float* dx32;
  float* doff;
};

template <typename T>
__global__ __launch_bounds__(256) void k_sample_bwd(const BwdParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x;
  const int lw = xcd_swizzle(blockIdx.x, p.num_wg);
  const int tile = lw / p.gsplit, gs = lw - tile * p.gsplit;
  const int tpi = p.tiles_h * p.tiles_w;
  const int n = tile / tpi, trem = tile - n * tpi;
  const int tyi = trem / p.tiles_w, txi = trem - tyi * p.tiles_w;
  const int oh0 = tyi * p.TH, ow0 = txi * p.TW;
  const int thn = min(p.TH, p.Ho - oh0), twn = min(p.TW, p.Wo - ow0);
  const int PT = p.TH * p.TW;
  const int g0 = gs * p.GW;
  const int ocw = 2 * p.GW * p.K2;
  const int obase = 2 * g0 * p.K2;
  T* xr = (T*)(smem + p.lds_x);
  float* dxr = (float*)(smem + p.lds_dx);
  float* off_l = (float*)(smem + p.lds_off);
  int4* info = (int4*)(smem + p.lds_info);
  float* doff_l = (float*)(smem + p.lds_doff);  // [GW][K2][PT][2]
  const T* __restrict__ x = (const T*)p.x;
  const T* __restrict__ dcol = (const T*)p.dcol;
  const int fy0 = oh0 * p.SH - p.PH, fx0 = ow0 * p.SW - p.PW;

  for (int e = tid; e < ocw * PT; e += 256) {
    const int o = e / PT, pix = e - o * PT;
    const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
    float v = 0.f;
    if (ty < thn && tx < twn) v = p.off[(((size_t)n * p.Oc + obase + o) * p.Ho + oh0 + ty) * p.Wo + ow0 + tx];
    off_l[e] = v;
  }
  for (int e = tid; e < p.GW * p.K2 * PT * 2; e += 256) doff_l[e] = 0.f;
  const int fha = (thn - 1) * p.SH + (p.KH - 1) * p.DH + 1;
  const int fwa = (twn - 1) * p.SW + (p.KW - 1) * p.DW + 1;
  const int ry0 = max(fy0 - p.halo, -1), ry1 = min(fy0 + fha + p.halo, p.H);
  const int rx0 = max(fx0 - p.halo, -1), rx1 = min(fx0 + fwa + p.halo, p.W);
  int RH = ry1 - ry0 + 1, RW = rx1 - rx0 + 1;
  if (RH <= 0 || RW <= 0) { RH = 0; RW = 0; }
  __syncthreads();
  for (int e = tid; e < p.GW * p.K2 * PT; e += 256) {
    const int gt = e / PT, pix = e - gt * PT;
    const int gl = fdiv(gt, p.div_k2), t = gt - gl * p.K2;
    const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
    int4 inf = make_int4(-2, 0, 0, 0);
    if (ty < thn && tx < twn) {
      const int ti = t / p.KW, tj = t - ti * p.KW;
      const int by = (oh0 + ty) * p.SH - p.PH + ti * p.DH;
      const int bx = (ow0 + tx) * p.SW - p.PW + tj * p.DW;
      const TapIndex ix = tap_index(by, bx, off_l[(2 * (gl * p.K2 + t)) * PT + pix],
                                    off_l[(2 * (gl * p.K2 + t) + 1) * PT + pix], p.H, p.W);
      if (!ix.outside) {
        const bool in = ix.y0 >= ry0 && ix.y0 + 1 <= ry1 && ix.x0 >= rx0 && ix.x0 + 1 <= rx1 && RH > 0;
        inf.x = in ? (ix.y0 - ry0) * RW + (ix.x0 - rx0) : -1;
        inf.y = (int)(((uint32_t)ix.y0 << 16) | ((uint32_t)ix.x0 & 0xffffu));
        inf.z = __float_as_int(ix.ly);
        inf.w = __float_as_int(ix.lx);
      }
    }
    info[e] = inf;
  }

  const FastDiv drw = make_fastdiv(RW > 0 ? RW : 1), drh = make_fastdiv(RH > 0 ? RH : 1);
  const int nv = p.CC >> 3;
  const int nitems = PT * p.K2 * nv;
  const size_t HW = (size_t)p.H * p.W;
  const int rtot = RH * RW;
  for (int gl = 0; gl < p.GW; ++gl) {
    const int g = g0 + gl;
    for (int c0 = 0; c0 < p.Cg; c0 += p.CC) {
      const int cglob = g * p.Cg + c0;
      __syncthreads();
      if (RH > 0) stage_region_hwc<T>(xr, x, p.Cin, p.H, p.W, n, cglob, p.CC, ry0, rx0, RH, RW, drw, drh, p.pstr);
      for (int e = tid; e < rtot * p.dstr; e += 256) dxr[e] = 0.f;
      __syncthreads();
      for (int it = tid; it < nitems; it += 256) {
        const int v = it & (nv - 1);
        const int rest = it >> p.lognv;
        const int pix = fdiv(rest, p.div_k2), t = rest - pix * p.K2;
        const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
        if (ty >= thn || tx >= twn) continue;
        const int4 inf = info[(gl * p.K2 + t) * PT + pix];
        float gy = 0.f, gx = 0.f;
        if (inf.x != -2) {
          const size_t q = (size_t)n * p.Ho * p.Wo + (size_t)(oh0 + ty) * p.Wo + (ow0 + tx);
          float gc[8];
          load8(dcol + q * p.Ck + (size_t)t * p.Cin + cglob + v * 8, gc);
          TapIndex ix;
          ix.outside = false;
          ix.ly = __int_as_float(inf.z);
          ix.lx = __int_as_float(inf.w);
          float w[4];
          tap_weights(ix, w);
          const float hy = 1.0f - ix.ly, hx = 1.0f - ix.lx;
          float f00[8], f01[8], f10[8], f11[8];
          if (inf.x >= 0) {
            const T* b0 = xr + (size_t)inf.x * p.pstr + v * 8;
            lds_read8(b0, f00);
            lds_read8(b0 + p.pstr, f01);
            lds_read8(b0 + (size_t)RW * p.pstr, f10);
            lds_read8(b0 + (size_t)(RW + 1) * p.pstr, f11);
            float* d0 = dxr + (size_t)inf.x * p.dstr + v * 8;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              atomicAdd(d0 + c, w[0] * gc[c]);
              atomicAdd(d0 + p.dstr + c, w[1] * gc[c]);
              atomicAdd(d0 + (size_t)RW * p.dstr + c, w[2] * gc[c]);
              atomicAdd(d0 + (size_t)(RW + 1) * p.dstr + c, w[3] * gc[c]);
            }
          } else {
            const int y0 = inf.y >> 16, x0 = (int)(short)(inf.y & 0xffff);
            const bool r0 = y0 >= 0, r1 = y0 + 1 < p.H, q0 = x0 >= 0, q1 = x0 + 1 < p.W;
            const T* base = x + ((size_t)n * p.Cin + cglob + v * 8) * HW;
            float* dbase = p.dx32 + ((size_t)n * p.Cin + cglob + v * 8) * HW;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const T* pl = base + c * HW;
              float* dl = dbase + c * HW;
              f00[c] = (r0 && q0) ? Elem<T>::to_f32(pl[(size_t)y0 * p.W + x0]) : 0.f;
              f01[c] = (r0 && q1) ? Elem<T>::to_f32(pl[(size_t)y0 * p.W + x0 + 1]) : 0.f;
              f10[c] = (r1 && q0) ? Elem<T>::to_f32(pl[(size_t)(y0 + 1) * p.W + x0]) : 0.f;
              f11[c] = (r1 && q1) ? Elem<T>::to_f32(pl[(size_t)(y0 + 1) * p.W + x0 + 1]) : 0.f;
              if (r0 && q0) atomicAdd(dl + (size_t)y0 * p.W + x0, w[0] * gc[c]);
              if (r0 && q1) atomicAdd(dl + (size_t)y0 * p.W + x0 + 1, w[1] * gc[c]);
              if (r1 && q0) atomicAdd(dl + (size_t)(y0 + 1) * p.W + x0, w[2] * gc[c]);
              if (r1 && q1) atomicAdd(dl + (size_t)(y0 + 1) * p.W + x0 + 1, w[3] * gc[c]);
            }
          }
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            gy = __builtin_fmaf(gc[c], hx * (f10[c] - f00[c]) + ix.lx * (f11[c] - f01[c]), gy);
            gx = __builtin_fmaf(gc[c], hy * (f01[c] - f00[c]) + ix.ly * (f11[c] - f10[c]), gx);
          }
        }
        // reduce over the nv lanes that share this (pixel, tap)
        for (int s = 1; s < nv; s <<= 1) {
          gy += __shfl_xor(gy, s);
          gx += __shfl_xor(gx, s);
        }
        if (v == 0) {
          float* dd = doff_l + ((gl * p.K2 + t) * PT + pix) * 2;
          dd[0] += gy;
          dd[1] += gx;
        }
      }
      __syncthreads();
      // add the region's dX to global memory (in-image pixels only)
      const int ntot = p.CC * rtot;
      for (int e = tid; e < ntot; e += 256) {
        const int r = fdiv(e, drw);
        const int rx = e - r * RW;
        const int c = fdiv(r, drh);
        const int ry = r - c * RH;
        const int yy = ry0 + ry, xx = rx0 + rx;
        if ((unsigned)yy < (unsigned)p.H && (unsigned)xx < (unsigned)p.W) {
          const float v = dxr[(ry * RW + rx) * p.dstr + c];
          if (v != 0.f) atomicAdd(p.dx32 + ((size_t)n * p.Cin + cglob + c) * HW + (size_t)yy * p.W + xx, v);
        }
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < p.GW * p.K2 * PT; e += 256) {
    const int gt = e / PT, pix = e - gt * PT;
    const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
    if (ty >= thn || tx >= twn) continue;
    const size_t base = (((size_t)n * p.Oc + obase + 2 * gt) * p.Ho + oh0 + ty) * p.Wo + ow0 + tx;
    p.doff[base] = doff_l[2 * e];
    p.doff[base + (size_t)p.Ho * p.Wo] = doff_l[2 * e + 1];
  }
}

// ---------------------------------------------------------------------------
// dW_off[o][t][c] += sum over output pixels of dOff[o][pix] * xz[c][tap t of
// pix].  GEMM with rows o (MB blocks of 32), columns (tap, channel) and depth
// pixels.  Workgroup = (image, 32-channel slice, band of output pixels); N
// block t of the GEMM is tap t for the slice's 32 channels, and wave w owns
// taps t = w, w+4, ...  Both operands are gathered from global memory (L2):
// A = 8 consecutive pixels of one dOff row, B = x at 8 consecutive pixels'
// tap-t positions for one channel.
struct WoffParams {
  int N, Cin, H, W, Ho, Wo, KH, KW, SH, SW, PH, PW, DH, DW, K2, Oc;
  int o0, orows;  // offset-channel rows [o0, o0+orows) handled by this launch (orows <= 96)
  int slices, bands, band_pix, num_wg;
  const void* x;
  const float* doff;
  float* dwoff32;  // [Oc][K2][Cin]
};

template <typename T, int MB>
__global__ __launch_bounds__(256) void k_woff_bwd(const WoffParams p) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int KC = 2 * VEC;  // pixels per k-chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lw = xcd_swizzle(blockIdx.x, p.num_wg);
  const int per_img = p.slices * p.bands;
  const int n = lw / per_img, r = lw - n * per_img;
  const int band = r / p.slices, cs = r - band * p.slices;
  const int HoWo = p.Ho * p.Wo;
  const int pb0 = band * p.band_pix, pb1 = min(HoWo, pb0 + p.band_pix);
  const int c = cs * 32 + (lane & 31);
  const bool cval = c < p.Cin;
  const int half = lane >> 5;
  const T* __restrict__ x = (const T*)p.x;
  const float* __restrict__ doff = p.doff + (size_t)n * p.Oc * HoWo;
  const T* xc = x + ((size_t)n * p.Cin + (cval ? c : 0)) * p.H * p.W;
  // taps are processed 12 at a time (3 per wave) so any kernel size fits
  for (int tg = 0; tg < p.K2; tg += 12) {
  f32x16_t acc[MB][3];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[mb][j][q] = 0.f;
  for (int k0 = pb0; k0 < pb1; k0 += KC) {
    const int kp = k0 + half * VEC;  // this lane's first pixel
    uint4 a[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int o = p.o0 + mb * 32 + (lane & 31);
      float f[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        f[e] = (o < p.o0 + p.orows && kp + e < pb1) ? doff[(size_t)o * HoWo + kp + e] : 0.f;
      if constexpr (VEC == 8) {
        a[mb] = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                           pack_bf16x2(f[6], f[7]));
      } else {
        a[mb] = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                           __float_as_uint(f[3]));
      }
    }
    int ho[VEC], wo[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int q = kp + e;
      ho[e] = q / p.Wo;
      wo[e] = q - ho[e] * p.Wo;
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int t = tg + wave + 4 * j;
      if (t >= p.K2) break;
      const int ti = t / p.KW, tj = t - ti * p.KW;
      float f[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int yy = ho[e] * p.SH - p.PH + ti * p.DH, xx = wo[e] * p.SW - p.PW + tj * p.DW;
        f[e] = (cval && kp + e < pb1 && (unsigned)yy < (unsigned)p.H && (unsigned)xx < (unsigned)p.W)
                   ? Elem<T>::to_f32(xc[(size_t)yy * p.W + xx])
                   : 0.f;
      }
      uint4 b;
      if constexpr (VEC == 8) {
        b = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                       pack_bf16x2(f[6], f[7]));
      } else {
        b = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) mfma_chunk(acc[mb][j], a[mb], b, T());
    }
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int t = tg + wave + 4 * j;
    if (t >= p.K2) break;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int o = p.o0 + mb * 32 + acc_row(lane, q);
        if (o < p.o0 + p.orows && cval) atomicAdd(p.dwoff32 + ((size_t)o * p.K2 + t) * p.Cin + c, acc[mb][j][q]);
      }
  }
  }
}

// ---------------------------------------------------------------------------
// dX_offset, the transposed offset convolution, plus the sampling part of dX
// accumulated so far, rounded once: dx[n][c][y][x] = dtype(dx32 + sum over
// (o, tap) of W_off[o][c][tap] * dOff[o][ho][wo]) with (y, x) the tap's grid
// position of (ho, wo).  GEMM with rows c (one 32-channel block per wave),
// columns = 64 input pixels, depth kk = o*K2 + tap (padded to KKP).  The B
// tile [pixel][kk] is built once per workgroup in LDS.
struct DxoffParams {
  int N, Cin, H, W, Ho, Wo, KH, KW, SH, SW, PH, PW, DH, DW, K2, Oc, KKP, KKC;
  int pix_blocks, cblocks, num_wg;
  const void* wofft;  // [Cin][KKP]
  const float* doff;
  const float* dx32;
  void* dx;
};

template <typename T>
__global__ __launch_bounds__(256) void k_dx_off(const DxoffParams p) {
  constexpr int VEC = Elem<T>::VEC;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lw = xcd_swizzle(blockIdx.x, p.num_wg);
  const int per_img = p.pix_blocks * p.cblocks;
  const int n = lw / per_img, r = lw - n * per_img;
  const int pbk = r / p.cblocks, cb = r - pbk * p.cblocks;
  const int HW = p.H * p.W, HoWo = p.Ho * p.Wo;
  const int pix0 = pbk * 64;
  const int bstr = p.KKC + VEC;  // LDS row stride (elements)
  T* bt = (T*)smem;              // [64][bstr]
  const float* __restrict__ doff = p.doff + (size_t)n * p.Oc * HoWo;
  const int c0 = cb * 128 + wave * 32;
  const bool active = c0 < p.Cin;
  const T* __restrict__ wt = (const T*)p.wofft;
  f32x16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[j][q] = 0.f;
  const int crow = c0 + (lane & 31);
  for (int kb = 0; kb < p.KKP; kb += p.KKC) {
    const int len = min(p.KKC, p.KKP - kb);
    __syncthreads();
    for (int e = tid; e < 64 * len; e += 256) {
      const int pix = e / len, kl = e - pix * len, kk = kb + kl;
      float v = 0.f;
      const int q = pix0 + pix;
      if (kk < p.Oc * p.K2 && q < HW) {
        const int o = kk / p.K2, t = kk - o * p.K2;
        const int ti = t / p.KW, tj = t - ti * p.KW;
        const int y = q / p.W, xx = q - y * p.W;
        const int ny = y + p.PH - ti * p.DH, nx = xx + p.PW - tj * p.DW;
        if (ny >= 0 && nx >= 0 && ny % p.SH == 0 && nx % p.SW == 0) {
          const int ho = ny / p.SH, wo = nx / p.SW;
          if (ho < p.Ho && wo < p.Wo) v = doff[(size_t)o * HoWo + (size_t)ho * p.Wo + wo];
        }
      }
      bt[pix * bstr + kl] = Elem<T>::from_f32(v);
    }
    __syncthreads();
    if (active) {
      const int nkc = len / (2 * VEC);
      for (int kc = 0; kc < nkc; ++kc) {
        const int kl = kc * 2 * VEC + (lane >> 5) * VEC;
        const uint4 a = crow < p.Cin ? *(const uint4*)(wt + (size_t)crow * p.KKP + kb + kl) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4 b = *(const uint4*)(bt + (j * 32 + (lane & 31)) * bstr + kl);
          mfma_chunk(acc[j], a, b, T());
        }
      }
    }
  }
  if (!active) return;
  T* dx = (T*)p.dx;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = pix0 + j * 32 + (lane & 31);
    if (q >= HW) continue;
#pragma unroll
    for (int r2 = 0; r2 < 16; ++r2) {
      const int cc = c0 + acc_row(lane, r2);
      if (cc < p.Cin) {
        const size_t idx = ((size_t)n * p.Cin + cc) * HW + q;
        dx[idx] = Elem<T>::from_f32(p.dx32[idx] + acc[j][r2]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prep: W2[(t,c)][co] = W[co][c][t]; WoffT[c][o*K2+t] = W_off[o][c][t] (zero
// for kk >= Oc*K2); fp32 accumulators zeroed.
template <typename T>
__global__ __launch_bounds__(256) void k_prep_backward(const T* __restrict__ w, const T* __restrict__ w_off, T* w2,
                                                       T* wofft, float* z0, size_t nz0, float* z1, size_t nz1,
                                                       float* z2, size_t nz2, int Cout, int Cin, int K2, int Oc,
                                                       int KKP) {
  const size_t n1 = (size_t)Cout * K2 * Cin, n2 = (size_t)Cin * KKP;
  const size_t total = n1 + n2 + nz0 + nz1 + nz2;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    if (e < n1) {
      const int co = (int)(e % Cout);
      const size_t r = e / Cout;
      const int c = (int)(r % Cin);
      const int t = (int)(r / Cin);
      w2[e] = w[((size_t)co * Cin + c) * K2 + t];
    } else if (e < n1 + n2) {
      const size_t f = e - n1;
      const int kk = (int)(f % KKP);
      const int c = (int)(f / KKP);
      wofft[f] = kk < Oc * K2 ? w_off[((size_t)(kk / K2) * Cin + c) * K2 + kk % K2] : zero_elem<T>();
    } else {
      size_t f = e - n1 - n2;
      if (f < nz0) { z0[f] = 0.f; continue; }
      f -= nz0;
      if (f < nz1) { z1[f] = 0.f; continue; }
      f -= nz1;
      z2[f] = 0.f;
    }
  }
}

// dw[co][c][t] = dtype(dw32[co][t][c]); dw_off likewise.
template <typename T>
__global__ __launch_bounds__(256) void k_finalize_w(const float* __restrict__ dw32, T* dw, int Cout,
                                                    const float* __restrict__ dwoff32, T* dwoff, int Oc, int Cin,
                                                    int K2) {
  const size_t n1 = (size_t)Cout * Cin * K2, n2 = (size_t)Oc * Cin * K2;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n1 + n2; e += (size_t)gridDim.x * 256) {
    const bool first = e < n1;
    const size_t f = first ? e : e - n1;
    const int t = (int)(f % K2);
    const size_t r = f / K2;
    const int c = (int)(r % Cin);
    const size_t o = r / Cin;
    const float v = (first ? dw32 : dwoff32)[(o * K2 + t) * Cin + c];
    (first ? dw : dwoff)[f] = Elem<T>::from_f32(v);
  }
}

// db[co] = sum over (n, pixel) of dY; db_off[o] = sum of dOff.  One workgroup
// per output channel, fixed-order tree reduction.
template <typename T>
__global__ __launch_bounds__(256) void k_bias_sums(const T* __restrict__ dy, T* db, int Cout, const float* __restrict__ doff,
                                                   T* dboff, int Oc, int N, int HoWo) {
  __shared__ float red[256];
  const int ch = blockIdx.x;
  const bool main = ch < Cout;
  if (main && !db) return;
  if (!main && !dboff) return;
  const int o = main ? ch : ch - Cout;
  const int C = main ? Cout : Oc;
  float s = 0.f;
  for (int n = 0; n < N; ++n) {
    const size_t base = ((size_t)n * C + o) * HoWo;
    for (int q = threadIdx.x; q < HoWo; q += 256)
      s += main ? Elem<T>::to_f32(dy[base + q]) : doff[base + q];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) (main ? db : dboff)[o] = Elem<T>::from_f32(red[0]);
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
  float* dx32 = (float*)(ws + p.ws_dx32);
  float* dw32 = (float*)(ws + p.ws_dw32);
  float* dwoff32 = (float*)(ws + p.ws_dwoff32);
  float* doff = (float*)(ws + p.ws_doff);
  const size_t ndx = (size_t)d.n * d.c_in * d.h * d.w;
  const size_t ndw = (size_t)d.c_out * p.ck, ndwoff = (size_t)p.oc * p.ck;
  {
    const size_t total = (size_t)d.c_out * p.ck + (size_t)d.c_in * p.kk_pad + ndx + ndw + ndwoff;
    DEFT_LAUNCH("prep_backward", k_prep_backward<T>, dim3(grid_cap(total, 8192)), dim3(256), 0, st, (const T*)a.w,
                       (const T*)a.w_off, w2, wofft, dx32, ndx, dw32, ndw, dwoff32, ndwoff, d.c_out, d.c_in,
                       p.taps, p.oc, p.kk_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_gemm_dcol(p, w2, a.dy, dcol, st);
  if (e != hipSuccess) return e;
  e = launch_gemm_dw(p, a.dy, cols, dw32, st);
  if (e != hipSuccess) return e;

  // sampling backward
  {
    BwdParams b;
    b.N = d.n; b.Cin = d.c_in; b.H = d.h; b.W = d.w; b.Ho = p.ho; b.Wo = p.wo; b.KH = d.kh; b.KW = d.kw;
    b.SH = d.stride_h; b.SW = d.stride_w; b.PH = d.pad_h; b.PW = d.pad_w; b.DH = d.dil_h; b.DW = d.dil_w;
    b.G = d.offset_groups; b.Cg = p.cg; b.K2 = p.taps; b.Oc = p.oc; b.Ck = p.ck; b.Cout = d.c_out;
    b.TH = p.tile_h; b.TW = p.tile_w; b.halo = p.halo; b.CC = p.chunk_b; b.GW = p.gw; b.gsplit = p.gsplit;
    b.tiles_h = p.tiles_h; b.tiles_w = p.tiles_w; b.num_wg = p.num_wg; b.FH = p.foot_h; b.FW = p.foot_w;
    b.pstr = p.pstr_b; b.dstr = p.dstr_b;
    int l = 0;
    while ((1 << l) < (p.chunk_b >> 3)) ++l;
    b.lognv = l;
    b.lds_x = p.lb_x; b.lds_dx = p.lb_dx; b.lds_off = p.lb_off; b.lds_info = p.lb_info; b.lds_doff = p.lb_doff;
    b.div_tw = make_fastdiv(p.tile_w); b.div_k2 = make_fastdiv(p.taps);
    b.x = a.x; b.off = a.offsets; b.dcol = dcol; b.dx32 = dx32; b.doff = doff;
    auto kern = k_sample_bwd<T>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, p.lb_total);
    if (e != hipSuccess) return e;
    if (p.num_wg) DEFT_LAUNCH("sample_backward", kern, dim3(p.num_wg), dim3(256), p.lb_total, st, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // offset-conv weight gradient
  {
    WoffParams w;
    w.N = d.n; w.Cin = d.c_in; w.H = d.h; w.W = d.w; w.Ho = p.ho; w.Wo = p.wo; w.KH = d.kh; w.KW = d.kw;
    w.SH = d.stride_h; w.SW = d.stride_w; w.PH = d.pad_h; w.PW = d.pad_w; w.DH = d.dil_h; w.DW = d.dil_w;
    w.K2 = p.taps; w.Oc = p.oc;
    w.slices = (d.c_in + 31) / 32;
    const int howo = p.ho * p.wo;
    int bands = 1;
    while (d.n * w.slices * bands < 256 && bands * 64 < howo) bands *= 2;
    const int kc = d.dtype == DEFT_BF16 ? 16 : 8;
    w.band_pix = ((howo + bands - 1) / bands + kc - 1) / kc * kc;
    w.bands = (howo + w.band_pix - 1) / w.band_pix;
    w.num_wg = d.n * w.slices * w.bands;
    w.x = a.x; w.doff = doff; w.dwoff32 = dwoff32;
    for (int o0 = 0; o0 < p.oc && w.num_wg; o0 += 96) {
      w.o0 = o0;
      w.orows = p.oc - o0 < 96 ? p.oc - o0 : 96;
      const int mb = (w.orows + 31) / 32;
      if (mb == 1) DEFT_LAUNCH("offset_weight_backward", (k_woff_bwd<T, 1>), dim3(w.num_wg), dim3(256), 0, st, w);
      else if (mb == 2) DEFT_LAUNCH("offset_weight_backward", (k_woff_bwd<T, 2>), dim3(w.num_wg), dim3(256), 0, st, w);
      else DEFT_LAUNCH("offset_weight_backward", (k_woff_bwd<T, 3>), dim3(w.num_wg), dim3(256), 0, st, w);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  // dX_offset + final dx
  {
    DxoffParams q;
    q.N = d.n; q.Cin = d.c_in; q.H = d.h; q.W = d.w; q.Ho = p.ho; q.Wo = p.wo; q.KH = d.kh; q.KW = d.kw;
    q.SH = d.stride_h; q.SW = d.stride_w; q.PH = d.pad_h; q.PW = d.pad_w; q.DH = d.dil_h; q.DW = d.dil_w;
    q.K2 = p.taps; q.Oc = p.oc; q.KKP = p.kk_pad;
    q.KKC = p.kk_pad < 256 ? p.kk_pad : 256;
    q.pix_blocks = (d.h * d.w + 63) / 64;
    q.cblocks = (d.c_in + 127) / 128;
    q.num_wg = d.n * q.pix_blocks * q.cblocks;
    q.wofft = wofft; q.doff = doff; q.dx32 = dx32; q.dx = a.dx;
    const int lds = 64 * (q.KKC + (d.dtype == DEFT_BF16 ? 8 : 4)) * (int)sizeof(T);
    auto kern = k_dx_off<T>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    if (q.num_wg) DEFT_LAUNCH("offset_input_backward", kern, dim3(q.num_wg), dim3(256), lds, st, q);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // weights and biases
  {
    const size_t total = ((size_t)d.c_out + p.oc) * d.c_in * p.taps;
    DEFT_LAUNCH("finalize_weights", k_finalize_w<T>, dim3(grid_cap(total, 4096)), dim3(256), 0, st, dw32, (T*)a.dw, d.c_out,
                       dwoff32, (T*)a.dw_off, p.oc, d.c_in, p.taps);
    if (a.db || a.db_off)
      DEFT_LAUNCH("bias_sums", k_bias_sums<T>, dim3(d.c_out + p.oc), dim3(256), 0, st, (const T*)a.dy, (T*)a.db, d.c_out,
                         doff, (T*)a.db_off, p.oc, d.n, p.ho * p.wo);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_backward(const deft_plan& p, const BackwardArgs& a, hipStream_t st) {
  return p.d.dtype == DEFT_BF16 ? backward_t<bf16_t>(p, a, st) : backward_t<float>(p, a, st);
}

}  // namespace deft
