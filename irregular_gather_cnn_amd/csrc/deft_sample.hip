// Fused offset convolution + bilinear sampling for gfx950.
//
// One workgroup owns one output tile (tile_h x tile_w pixels of one image)
// and a slice of the offset groups.  Phase A computes that tile's offsets as
// an implicit GEMM on the MFMA units (rows: offset channels; columns: tile
// pixels; depth: taps x input channels read from the tile's footprint staged
// in LDS) and keeps them in LDS; phase B computes each tap's integer corner
// and fractional weights once, then, one channel chunk at a time, stages the
// footprint plus a halo of the input in LDS (channel-minor, so a lane reads 8
// channels of a corner as one 16-byte word), blends the four corners and
// writes the deformed columns.  Taps whose corners fall outside the halo read
// the input from global memory.  This follows the DefT explainer page ("How
// DefT works", "The idea"; "Why it works"): the offset convolution and the
// interpolation share the input, so fusing them keeps the offsets on chip and
// reuses the staged input; tiling by the output's spatial dimensions puts the
// gathers in on-chip memory; a halo sized from the offset distribution keeps
// out-of-tile accesses rare.  The workgroup order is XCD-aware so tiles that
// share halo rows run on the same XCD's L2 (the page's block-ID swizzle).
#include "deft_device.h"
#include "deft_internal.h"

namespace deft {

struct SampleParams {
  int N, Cin, H, W, Ho, Wo, KH, KW, SH, SW, PH, PW, DH, DW, G, Cg, K2, Oc, Ck;
  int TH, TW, halo, CC, CA, GW, gsplit, tiles_h, tiles_w, num_wg;
  int FH, FW, pstr, pstr_a, lognv;
  int lds_region, lds_off, lds_info;
  FastDiv div_tw, div_k2, div_fh;
  const void* x;
  const void* woff_p;
  const void* b_off;
  const float* off_in;
  float* off_out;
  void* cols;
};

template <typename T, bool FUSED, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_sample(const SampleParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int VEC = Elem<T>::VEC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  float* off_l = (float*)(smem + p.lds_off);   // [ocw][PT]
  int2* tab = (int2*)(smem + p.lds_info);                            // [GW][PT][K2]
  float4* wts = (float4*)(smem + p.lds_info + ((p.GW * PT * p.K2 * 8 + 15) & ~15));  // [GW][PT][K2]
  T* xr = (T*)(smem + p.lds_region);
  const T* __restrict__ x = (const T*)p.x;
  const int fy0 = oh0 * p.SH - p.PH, fx0 = ow0 * p.SW - p.PW;

  // ---- halo region of this tile (clipped to rows/cols -1..H, -1..W) ----
  const int fha = (thn - 1) * p.SH + (p.KH - 1) * p.DH + 1;
  const int fwa = (twn - 1) * p.SW + (p.KW - 1) * p.DW + 1;
  const int ry0 = max(fy0 - p.halo, -1), ry1 = min(fy0 + fha + p.halo, p.H);
  const int rx0 = max(fx0 - p.halo, -1), rx1 = min(fx0 + fwa + p.halo, p.W);
  int RH = ry1 - ry0 + 1, RW = rx1 - rx0 + 1;
  if (RH <= 0 || RW <= 0) { RH = 0; RW = 0; }

  // Input staging: bf16 with an even width goes through registers so the next
  // chunk's loads overlap the current chunk's compute (kItemsA / kItemsB
  // items of 8 channels x 2 pixels per thread for the footprint / halo
  // chunks); larger regions and other inputs are staged synchronously.
  constexpr int kItemsA = 3, kItemsB = 8;
  const size_t img_elems = (size_t)p.Cin * p.H * p.W;
  const bool pairs_ok = sizeof(T) == 2 && (p.W & 1) == 0 && img_elems < 0x3ffffff0u;
  const PairGeom gb = pair_geom(p.H, p.W, p.CC, ry0, rx0, RH, RW, p.pstr);
  const bool pipeB = pairs_ok && RH > 0 && gb.total <= 256 * kItemsB;
  const __amdgpu_buffer_rsrc_t ximg = make_brsrc(x + (size_t)n * img_elems, pairs_ok ? (uint32_t)(img_elems * 2) : 0u);
  PairStage<kItemsB> st;

  if constexpr (FUSED) {
    // ---- phase A: offsets of this tile on the MFMA units ----
    f32x16_t acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
    const int nkc = p.CA / (2 * VEC);
    const int npairs = p.K2 * nkc;
    const int myp = (npairs - wave + 3) >> 2;  // this wave's (tap, k-chunk) pairs: wave, wave+4, ...
    const bool nb1 = PT > 32;
    const T* __restrict__ wp = (const T*)p.woff_p;
    int pixb[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      int pix = nb * 32 + (lane & 31);
      if (pix >= PT) pix = 0;
      const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
      pixb[nb] = ty * p.SH * p.FW + tx * p.SW;  // footprint pixel of tap (0,0)
    }
    const StageGeom sga = stage_geom<T>(p.W, fx0, p.FW, img_elems);
    const PairGeom ga = pair_geom(p.H, p.W, p.CA, fy0, fx0, p.FH, p.FW, p.pstr_a);
    const bool pipeA = pairs_ok && ga.total <= 256 * kItemsA;
    PairStage<kItemsA> sa;
    if (pipeA) pair_load(sa, ga, ximg, 0);
    // Weight fragments of this wave, a batch of kWB pairs at a time; the
    // first batch of the next chunk is loaded while this chunk computes.
    constexpr int kWB = 9 / MB;
    uint4 wa[kWB][MB], wn[kWB][MB];
    auto load_w = [&](uint4 (&dst)[kWB][MB], int c0, int j0) {
#pragma unroll
      for (int jj = 0; jj < kWB; ++jj) {
        const int j = j0 + jj;
        if (j < myp) {
          const int pi = wave + 4 * j;
          const int t = pi / nkc, kc = pi - t * nkc;
          const int cl = kc * 2 * VEC + (lane >> 5) * VEC;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int o = obase + mb * 32 + (lane & 31);
            dst[jj][mb] = *(const uint4*)(wp + ((size_t)o * p.K2 + t) * p.Cin + c0 + cl);
          }
        }
      }
    };
    load_w(wa, 0, 0);
    for (int c0 = 0; c0 < p.Cin; c0 += p.CA) {
      __syncthreads();
      if (pipeA) pair_store(sa, ga, (bf16_t*)xr);
      else stage_region<T>(xr, x, p.Cin, p.H, p.W, n, c0, p.CA, fy0, fx0, p.FH, p.FW, p.div_fh, sga, p.pstr_a);
      __syncthreads();
      const bool more = c0 + p.CA < p.Cin;
      if (pipeA && more) pair_load(sa, ga, ximg, c0 + p.CA);
      if (more) load_w(wn, c0 + p.CA, 0);
      for (int j0 = 0; j0 < myp; j0 += kWB) {
        if (j0 > 0) load_w(wa, c0, j0);
#pragma unroll
        for (int jj = 0; jj < kWB; ++jj) {
          const int j = j0 + jj;
          if (j >= myp) break;
          const int pi = wave + 4 * j;
          const int t = pi / nkc, kc = pi - t * nkc;
          const int ti = t / p.KW, tj = t - ti * p.KW;
          const int cl = kc * 2 * VEC + (lane >> 5) * VEC;
          const int toff = ti * p.DH * p.FW + tj * p.DW;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            if (nb == 1 && !nb1) break;
            const uint4 bq = *(const uint4*)(xr + (size_t)(pixb[nb] + toff) * p.pstr_a + cl);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) mfma_chunk(acc[mb][nb], wa[jj][mb], bq, T());
          }
        }
      }
      if (more) {
#pragma unroll
        for (int jj = 0; jj < kWB; ++jj)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) wa[jj][mb] = wn[jj][mb];
      }
    }
    __syncthreads();
    float* part = (float*)(smem + p.lds_region);  // [4][ocw][PT]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mb * 32 + acc_row(lane, r), col = nb * 32 + (lane & 31);
          if (row < ocw && col < PT) part[(wave * ocw + row) * PT + col] = acc[mb][nb][r];
        }
    __syncthreads();
    const int tot = ocw * PT;
    for (int e = tid; e < tot; e += 256) {
      const int o = e / PT, pix = e - o * PT;
      float v = part[e] + part[tot + e];
      v += part[2 * tot + e];
      v += part[3 * tot + e];
      if (p.b_off) v += Elem<T>::to_f32(((const T*)p.b_off)[obase + o]);
      off_l[e] = v;
      const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
      if (p.off_out && ty < thn && tx < twn)
        p.off_out[(((size_t)n * p.Oc + obase + o) * p.Ho + oh0 + ty) * p.Wo + ow0 + tx] = v;
    }
  } else {
    const int tot = ocw * PT;
    for (int e = tid; e < tot; e += 256) {
      const int o = e / PT, pix = e - o * PT;
      const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
      float v = 0.f;
      if (ty < thn && tx < twn)
        v = p.off_in[(((size_t)n * p.Oc + obase + o) * p.Ho + oh0 + ty) * p.Wo + ow0 + tx];
      off_l[e] = v;
    }
  }

  if (pipeB) pair_load(st, gb, ximg, g0 * p.Cg);  // first halo chunk, in flight during the index stage
  __syncthreads();

  // ---- tap index stage: once per (group, pixel, tap) ----
  // tab[e] = {corner (y0, x0) as an element offset into the staged region,
  // or -2 fully outside, <= -3 corner outside the halo (then
  // -3 - ((y0+1)*(W+1) + (x0+1))); column offset of the tap relative to the
  // tile's first column row, -1 for pixels outside the tile}; wts[e] = the
  // four bilinear weights.  e = (group*PT + pixel)*K2 + tap.
  const int nent = PT * p.K2;
  const int rwp = RW * p.pstr;
  {
    const int nidx = p.GW * nent;
    for (int e = tid; e < nidx; e += 256) {
      const int r = fdiv(e, p.div_k2), t = e - r * p.K2;
      const int gl = r / PT, pix = r - gl * PT;
      const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
      int2 tb = make_int2(0, -1);
      float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ty < thn && tx < twn) {
        const int ti = t / p.KW, tj = t - ti * p.KW;
        const int by = (oh0 + ty) * p.SH - p.PH + ti * p.DH;
        const int bx = (ow0 + tx) * p.SW - p.PW + tj * p.DW;
        const float dy = off_l[(2 * (gl * p.K2 + t)) * PT + pix];
        const float dx = off_l[(2 * (gl * p.K2 + t) + 1) * PT + pix];
        const TapIndex ix = tap_index(by, bx, dy, dx, p.H, p.W);
        tb.y = (ty * p.Wo + tx) * p.Ck + t * p.Cin;
        if (ix.outside) {
          tb.x = -2;
        } else {
          const bool in = ix.y0 >= ry0 && ix.y0 + 1 <= ry1 && ix.x0 >= rx0 && ix.x0 + 1 <= rx1 && RH > 0;
          tb.x = in ? ((ix.y0 - ry0) * RW + (ix.x0 - rx0)) * p.pstr : -3 - ((ix.y0 + 1) * (p.W + 1) + (ix.x0 + 1));
          float w[4];
          tap_weights(ix, w);
          wv = make_float4(w[0], w[1], w[2], w[3]);
        }
      }
      tab[e] = tb;
      wts[e] = wv;
    }
  }

  // ---- phase B: stage chunk + halo, blend four corners, write columns ----
  // Each thread keeps one 8-channel slice v of the chunk and walks the
  // (pixel, tap) entries; the nv threads of an entry write its chunk as one
  // contiguous run of the column row.
  const FastDiv drh = make_fastdiv(RH > 0 ? RH : 1);
  const StageGeom sg = stage_geom<T>(p.W, rx0, RW, img_elems);
  T* __restrict__ colt = (T*)p.cols + ((size_t)n * p.Ho * p.Wo + (size_t)oh0 * p.Wo + ow0) * p.Ck;
  const int nv = p.CC >> 3;
  const int v = tid & (nv - 1), e0 = tid >> p.lognv, estep = 256 >> p.lognv;
  const size_t HW = (size_t)p.H * p.W;
  for (int gl = 0; gl < p.GW; ++gl) {
    const int g = g0 + gl;
    const int2* tabg = tab + gl * nent;
    const float4* wtsg = wts + gl * nent;
    for (int c0 = 0; c0 < p.Cg; c0 += p.CC) {
      const int cglob = g * p.Cg + c0;
      __syncthreads();
      if (pipeB) pair_store(st, gb, (bf16_t*)xr);
      else if (RH > 0) stage_region<T>(xr, x, p.Cin, p.H, p.W, n, cglob, p.CC, ry0, rx0, RH, RW, drh, sg, p.pstr);
      __syncthreads();
      if (pipeB) {
        // next halo chunk: same group, next channels, else the next group
        const int cn = c0 + p.CC < p.Cg ? cglob + p.CC : (gl + 1 < p.GW ? (g + 1) * p.Cg : -1);
        if (cn >= 0) pair_load(st, gb, ximg, cn);
      }
      const T* xv = xr + v * 8;
      T* colv = colt + cglob + v * 8;
      // Every entry is blended from the staged region; entries that are fully
      // outside or whose
      // corner lies beyond the halo read corner 0 and are rewritten below by
      // the same thread.
      constexpr int kE = 1;  // entries per step (registers: the next chunk's loads are live here)
      for (int e = e0; e < nent; e += kE * estep) {
        int2 tb[kE];
        float w[kE][4];
#pragma unroll
        for (int u = 0; u < kE; ++u) {
          const int eu = e + u * estep;
          const int ec = eu < nent ? eu : e;
          tb[u] = tabg[ec];
          if (eu >= nent) tb[u].y = -1;
          const float4 wq = wtsg[ec];
          w[u][0] = wq.x; w[u][1] = wq.y; w[u][2] = wq.z; w[u][3] = wq.w;
        }
        float o8[kE][8];
#pragma unroll
        for (int u = 0; u < kE; ++u) {
          const T* b0 = xv + max(tb[u].x, 0);
          float f00[8], f01[8], f10[8], f11[8];
          lds_read8(b0, f00);
          lds_read8(b0 + p.pstr, f01);
          lds_read8(b0 + rwp, f10);
          lds_read8(b0 + rwp + p.pstr, f11);
#pragma unroll
          for (int c = 0; c < 8; ++c) o8[u][c] = blend4(w[u], f00[c], f01[c], f10[c], f11[c]);
        }
#pragma unroll
        for (int u = 0; u < kE; ++u)
          if (tb[u].y >= 0) store8(colv + tb[u].y, o8[u]);
      }
      // fully outside taps (zero) and corners beyond the halo (global reads)
      for (int e = e0; e < nent; e += estep) {
        const int2 tb = tabg[e];
        if (tb.x >= 0 || tb.y < 0) continue;
        float o8[8];
        if (tb.x == -2) {
#pragma unroll
          for (int c = 0; c < 8; ++c) o8[c] = 0.f;
        } else {
          const float4 wq = wtsg[e];
          const float w[4] = {wq.x, wq.y, wq.z, wq.w};
          const int m = -3 - tb.x;
          const int yy = m / (p.W + 1), y0 = yy - 1, x0 = m - yy * (p.W + 1) - 1;
          const bool r0 = y0 >= 0, r1 = y0 + 1 < p.H, q0 = x0 >= 0, q1 = x0 + 1 < p.W;
          const T* base = x + ((size_t)n * p.Cin + cglob + v * 8) * HW;
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const T* pl = base + c * HW;
            const float v00 = (r0 && q0) ? Elem<T>::to_f32(pl[(size_t)y0 * p.W + x0]) : 0.f;
            const float v01 = (r0 && q1) ? Elem<T>::to_f32(pl[(size_t)y0 * p.W + x0 + 1]) : 0.f;
            const float v10 = (r1 && q0) ? Elem<T>::to_f32(pl[(size_t)(y0 + 1) * p.W + x0]) : 0.f;
            const float v11 = (r1 && q1) ? Elem<T>::to_f32(pl[(size_t)(y0 + 1) * p.W + x0 + 1]) : 0.f;
            o8[c] = blend4(w, v00, v01, v10, v11);
          }
        }
        store8(colv + tb.y, o8);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tap index / corner mask on its own (same tap_index as the fused kernel).
struct IndexParams {
  int N, H, W, Ho, Wo, KH, KW, SH, SW, PH, PW, DH, DW, G, K2, Oc;
};
__global__ __launch_bounds__(256) void k_sample_index(const IndexParams p, const float* __restrict__ off,
                                                      int32_t* y0o, int32_t* x0o, uint8_t* mo) {
  const size_t total = (size_t)p.N * p.G * p.K2 * p.Ho * p.Wo;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    size_t r = e;
    const int wo = (int)(r % p.Wo); r /= p.Wo;
    const int ho = (int)(r % p.Ho); r /= p.Ho;
    const int t = (int)(r % p.K2); r /= p.K2;
    const int g = (int)(r % p.G);
    const int n = (int)(r / p.G);
    const int ti = t / p.KW, tj = t % p.KW;
    const size_t ob = ((size_t)n * p.Oc + 2 * (g * p.K2 + t)) * p.Ho * p.Wo + (size_t)ho * p.Wo + wo;
    const TapIndex ix = tap_index(ho * p.SH - p.PH + ti * p.DH, wo * p.SW - p.PW + tj * p.DW, off[ob],
                                  off[ob + (size_t)p.Ho * p.Wo], p.H, p.W);
    y0o[e] = ix.y0;
    x0o[e] = ix.x0;
    mo[e] = (uint8_t)corner_mask(ix, p.H, p.W);
  }
}

// Required-halo histogram: bin = Chebyshev distance of corner (y0, x0) from
// the tap's grid position, saturated at hist_len-2; fully outside taps go to
// bin hist_len-1.
__global__ __launch_bounds__(256) void k_halo_hist(const IndexParams p, const float* __restrict__ off,
                                                   uint32_t* hist, int hist_len) {
  __shared__ uint32_t h[64];
  for (int i = threadIdx.x; i < 64; i += 256) h[i] = 0;
  __syncthreads();
  const size_t total = (size_t)p.N * p.G * p.K2 * p.Ho * p.Wo;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    size_t r = e;
    const int wo = (int)(r % p.Wo); r /= p.Wo;
    const int ho = (int)(r % p.Ho); r /= p.Ho;
    const int t = (int)(r % p.K2); r /= p.K2;
    const int g = (int)(r % p.G);
    const int n = (int)(r / p.G);
    const int ti = t / p.KW, tj = t % p.KW;
    const int by = ho * p.SH - p.PH + ti * p.DH, bx = wo * p.SW - p.PW + tj * p.DW;
    const size_t ob = ((size_t)n * p.Oc + 2 * (g * p.K2 + t)) * p.Ho * p.Wo + (size_t)ho * p.Wo + wo;
    const TapIndex ix = tap_index(by, bx, off[ob], off[ob + (size_t)p.Ho * p.Wo], p.H, p.W);
    int bin;
    if (ix.outside) {
      bin = hist_len - 1;
    } else {
      const int dyv = abs(ix.y0 - by), dxv = abs(ix.x0 - bx);
      bin = min(max(dyv, dxv), hist_len - 2);
    }
    atomicAdd(&h[bin], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < hist_len; i += 256)
    if (h[i]) atomicAdd(&hist[i], h[i]);
}

__global__ void k_fill_u32(uint32_t* p, int n, uint32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Weight preparation: main weight [Cout][Cin][K] -> [Cout][K][Cin] (the
// column order) and offset-conv weight [Oc][Cin][K] -> [oc_pad][K][Cin],
// rows >= Oc zero.
template <typename T>
__global__ __launch_bounds__(256) void k_prep_forward(const T* __restrict__ w, const T* __restrict__ w_off,
                                                      T* wt, T* woff_p, int Cout, int Cin, int K2, int Oc,
                                                      int OcP) {
  const size_t n1 = (size_t)Cout * K2 * Cin, n2 = (size_t)OcP * K2 * Cin;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < n1 + n2; e += (size_t)gridDim.x * 256) {
    if (e < n1) {
      const int c = (int)(e % Cin);
      const size_t r = e / Cin;
      const int t = (int)(r % K2);
      const int co = (int)(r / K2);
      wt[e] = w[((size_t)co * Cin + c) * K2 + t];
    } else {
      const size_t f = e - n1;
      const int c = (int)(f % Cin);
      const size_t r = f / Cin;
      const int t = (int)(r % K2);
      const int o = (int)(r / K2);
      woff_p[f] = o < Oc ? w_off[((size_t)o * Cin + c) * K2 + t] : zero_elem<T>();
    }
  }
}

// ---------------------------------------------------------------------------
static SampleParams make_params(const deft_plan& p, const SampleArgs& a) {
  const deft_desc& d = p.d;
  SampleParams s;
  s.N = d.n; s.Cin = d.c_in; s.H = d.h; s.W = d.w; s.Ho = p.ho; s.Wo = p.wo;
  s.KH = d.kh; s.KW = d.kw; s.SH = d.stride_h; s.SW = d.stride_w; s.PH = d.pad_h; s.PW = d.pad_w;
  s.DH = d.dil_h; s.DW = d.dil_w; s.G = d.offset_groups; s.Cg = p.cg; s.K2 = p.taps; s.Oc = p.oc;
  s.Ck = p.ck;
  s.TH = p.tile_h; s.TW = p.tile_w; s.halo = p.halo; s.CC = p.chunk; s.CA = p.chunk_a; s.GW = p.gw;
  s.gsplit = p.gsplit; s.tiles_h = p.tiles_h; s.tiles_w = p.tiles_w; s.num_wg = p.num_wg;
  s.FH = p.foot_h; s.FW = p.foot_w; s.pstr = p.pstr; s.pstr_a = p.pstr_a;
  int l = 0;
  while ((1 << l) < (p.chunk >> 3)) ++l;
  s.lognv = l;
  s.lds_region = p.lds_region; s.lds_off = p.lds_off; s.lds_info = p.lds_info;
  s.div_tw = make_fastdiv(p.tile_w);
  s.div_k2 = make_fastdiv(p.taps);
  s.div_fh = make_fastdiv(p.foot_h);
  s.x = a.x; s.woff_p = a.woff_p; s.b_off = a.b_off; s.off_in = a.off_in; s.off_out = a.off_out;
  s.cols = a.cols;
  return s;
}

template <typename T, bool FUSED, int MB>
static hipError_t launch_sample_t(const deft_plan& p, const SampleParams& s, hipStream_t st) {
  auto kern = k_sample<T, FUSED, MB>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_total);
  if (e != hipSuccess) return e;
  DEFT_LAUNCH(FUSED ? "fused_offset_sample" : "sample_only", kern, dim3(p.num_wg), dim3(256), p.lds_total, st, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_sample_dt(const deft_plan& p, bool fused, const SampleParams& s, hipStream_t st) {
  if (!fused) return launch_sample_t<T, false, 1>(p, s, st);
  switch (p.mblocks) {
    case 1: return launch_sample_t<T, true, 1>(p, s, st);
    case 2: return launch_sample_t<T, true, 2>(p, s, st);
    case 3: return launch_sample_t<T, true, 3>(p, s, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sample(const deft_plan& p, bool fused, const SampleArgs& a, hipStream_t st) {
  const SampleParams s = make_params(p, a);
  if (p.num_wg == 0) return hipSuccess;
  return p.d.dtype == DEFT_BF16 ? launch_sample_dt<bf16_t>(p, fused, s, st)
                                : launch_sample_dt<float>(p, fused, s, st);
}

static IndexParams make_index_params(const deft_desc& d, int ho, int wo) {
  IndexParams s;
  s.N = d.n; s.H = d.h; s.W = d.w; s.Ho = ho; s.Wo = wo; s.KH = d.kh; s.KW = d.kw;
  s.SH = d.stride_h; s.SW = d.stride_w; s.PH = d.pad_h; s.PW = d.pad_w; s.DH = d.dil_h; s.DW = d.dil_w;
  s.G = d.offset_groups; s.K2 = d.kh * d.kw; s.Oc = 2 * s.G * s.K2;
  return s;
}

static unsigned grid_for(size_t total) {
  size_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  return (unsigned)(g ? g : 1);
}

hipError_t launch_sample_index(const deft_desc& d, int ho, int wo, const float* off, int32_t* y0,
                               int32_t* x0, uint8_t* mask, hipStream_t st) {
  const IndexParams s = make_index_params(d, ho, wo);
  const size_t total = (size_t)s.N * s.G * s.K2 * ho * wo;
  if (total == 0) return hipSuccess;
  DEFT_LAUNCH("index_stage", k_sample_index, dim3(grid_for(total)), dim3(256), 0, st, s, off, y0, x0, mask);
  return hipGetLastError();
}

hipError_t launch_halo_hist(const deft_desc& d, int ho, int wo, const float* off, uint32_t* hist,
                            int hist_len, hipStream_t st) {
  const IndexParams s = make_index_params(d, ho, wo);
  DEFT_LAUNCH("fill", k_fill_u32, dim3((hist_len + 255) / 256), dim3(256), 0, st, hist, hist_len, 0u);
  const size_t total = (size_t)s.N * s.G * s.K2 * ho * wo;
  if (total) {
    unsigned g = grid_for(total);
    if (g > 2048) g = 2048;
    DEFT_LAUNCH("halo_hist", k_halo_hist, dim3(g), dim3(256), 0, st, s, off, hist, hist_len);
  }
  return hipGetLastError();
}

hipError_t launch_prep_forward(const deft_plan& p, const void* w, const void* w_off, void* wt,
                               void* woff_p, hipStream_t st) {
  const deft_desc& d = p.d;
  const size_t total = (size_t)(d.c_out + p.oc_pad) * p.taps * d.c_in;
  unsigned g = grid_for(total);
  if (g > 4096) g = 4096;
  if (d.dtype == DEFT_BF16)
    DEFT_LAUNCH("prep_forward", k_prep_forward<bf16_t>, dim3(g), dim3(256), 0, st, (const bf16_t*)w,
                       (const bf16_t*)w_off, (bf16_t*)wt, (bf16_t*)woff_p, d.c_out, d.c_in, p.taps, p.oc,
                       p.oc_pad);
  else
    DEFT_LAUNCH("prep_forward", k_prep_forward<float>, dim3(g), dim3(256), 0, st, (const float*)w,
                       (const float*)w_off, (float*)wt, (float*)woff_p, d.c_out, d.c_in, p.taps, p.oc,
                       p.oc_pad);
  return hipGetLastError();
}

}  // namespace deft
