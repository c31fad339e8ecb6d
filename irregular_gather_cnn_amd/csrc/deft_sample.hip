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
// A second variant (k_sample_direct, bf16) reads every corner straight from a
// channel-minor copy of the input held in the caches instead of an LDS halo;
// its phase A stages only the footprint, by direct buffer-to-LDS loads.
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
  const void* xh;    // direct path: x channel-minor [N][H*W+1][Cin] (dtype), pixel H*W = 0
  int nv_log;        // direct path: log2(Cg / 8)
  int offsets_only;  // 1: stop after the offset convolution (offsets written to off_out)
  uint32_t* hist;    // nullable: the tile's required-halo histogram is added here
  int hist_len;      // 3..64 bins when hist is given
  int stage_d;       // direct path: footprint-staging loads per wave per chunk
  FastDiv div_fw;
};

// Phase-A work split.  The offset convolution's depth (taps x input
// channels) is cut into units of one tap x one chunk of CA channels, unit
// u = chunk * K2 + tap, and wave w takes units w, w + 4, w + 8, ...  Inside a
// unit the depth goes in k-steps of one MFMA; at step s lane half h holds the
// VEC channels chunk * CA + h * CA / 2 + s * VEC (the A and B operands use the
// same assignment), so over a unit each lane reads one contiguous run of CA/2
// channels of its pixel or offset channel: whole cache lines per wave.  Steps
// go in batches of up to four.  Both sampling kernels use this walk, so they
// accumulate identical products in identical order (bit-identical offsets).
struct UnitWalk {
  int c, t, kb;  // chunk, tap, first k-step of the batch
  __device__ __forceinline__ void start(int wave, int K2) {
    c = 0; t = wave; kb = 0;
    while (t >= K2) { t -= K2; ++c; }
  }
  __device__ __forceinline__ void next(int K2, int nks) {
    kb += 4;
    if (kb >= nks) {
      kb = 0; t += 4;
      while (t >= K2) { t -= K2; ++c; }
    }
  }
};

// Adds the required-halo histogram of this tile's taps to p.hist (the bins
// of deft_halo_histogram: Chebyshev distance from the tap's grid point to its
// corner (y0, x0), the last bin for fully outside taps), from the offsets in
// LDS (off_l [2 * gw * K2][PT]).  The emitted distribution is what the
// planner sizes the halo from (DefT page, "What to keep in mind": the gains
// depend on the offset distribution, so it is observed as the layer runs).
// Each wave counts its entries with one ballot per bin (lane b keeps bin b)
// and adds its counts with at most hist_len global atomics.  Called by all
// threads; the loop over entries is uniform within each wave.
__device__ __forceinline__ void tile_halo_hist(const SampleParams& p, const float* off_l, int gw, int oh0, int ow0,
                                            int thn, int twn) {
  const int lane = threadIdx.x & 63;
  const int PT = p.TH * p.TW, nidx = gw * PT * p.K2;
  uint32_t cnt = 0;
  for (int eb = (int)threadIdx.x - lane; eb < nidx; eb += (int)blockDim.x) {
    const int e = eb + lane;
    int bin = -1;
    if (e < nidx) {
      const int r = e / p.K2, t = e - r * p.K2;
      const int gl = r / PT, pix = r - gl * PT;
      const int ty = pix / p.TW, tx = pix - ty * p.TW;
      if (ty < thn && tx < twn) {
        const int ti = t / p.KW, tj = t - ti * p.KW;
        const int by = (oh0 + ty) * p.SH - p.PH + ti * p.DH;
        const int bx = (ow0 + tx) * p.SW - p.PW + tj * p.DW;
        const float dy = off_l[(2 * (gl * p.K2 + t)) * PT + pix];
        const float dx = off_l[(2 * (gl * p.K2 + t) + 1) * PT + pix];
        const TapIndex ix = tap_index(by, bx, dy, dx, p.H, p.W);
        bin = ix.outside ? p.hist_len - 1 : min(max(abs(ix.y0 - by), abs(ix.x0 - bx)), p.hist_len - 2);
      }
    }
    for (int b = 0; b < p.hist_len; ++b) {
      const uint64_t m = __ballot(bin == b);
      if (lane == b) cnt += (uint32_t)__popcll(m);
    }
  }
  if (lane < p.hist_len && cnt) atomicAdd(&p.hist[lane], cnt);
}

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
    const int nks = p.CA / (2 * VEC), nch = p.Cin / p.CA;
    const int hoff = (lane >> 5) * (p.CA / 2);
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
    // Weight fragments of one batch of k-steps; the next batch's are loaded
    // while this one computes.
    uint4 wa[4][MB], wn[4][MB];
    auto load_w = [&](uint4 (&dst)[4][MB], const UnitWalk& u) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (u.kb + k < nks) {
          const int cl = u.c * p.CA + hoff + (u.kb + k) * VEC;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            const int o = obase + mb * 32 + (lane & 31);
            dst[k][mb] = *(const uint4*)(wp + ((size_t)o * p.K2 + u.t) * p.Cin + cl);
          }
        }
      }
    };
    UnitWalk uw;
    uw.start(wave, p.K2);
    if (uw.c < nch) load_w(wa, uw);
    for (int c = 0; c < nch; ++c) {
      const int c0 = c * p.CA;
      __syncthreads();
      if (pipeA) pair_store(sa, ga, (bf16_t*)xr);
      else stage_region<T>(xr, x, p.Cin, p.H, p.W, n, c0, p.CA, fy0, fx0, p.FH, p.FW, p.div_fh, sga, p.pstr_a);
      __syncthreads();
      if (pipeA && c + 1 < nch) pair_load(sa, ga, ximg, c0 + p.CA);
      while (uw.c == c) {
        UnitWalk un = uw;
        un.next(p.K2, nks);
        if (un.c < nch) load_w(wn, un);
        const int ti = uw.t / p.KW, tj = uw.t - ti * p.KW;
        const int toff = ti * p.DH * p.FW + tj * p.DW;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (uw.kb + k >= nks) break;
          const int cl = hoff + (uw.kb + k) * VEC;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            if (nb == 1 && !nb1) break;
            const uint4 bq = *(const uint4*)(xr + (size_t)(pixb[nb] + toff) * p.pstr_a + cl);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) mfma_chunk(acc[mb][nb], wa[k][mb], bq, T());
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) wa[k][mb] = wn[k][mb];
        uw = un;
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
    if (p.offsets_only) {  // uniform: the whole workgroup leaves together
      // (the histogram of the offsets it computed still counts)
      if (p.hist) {
        __syncthreads();
        tile_halo_hist(p, off_l, p.GW, oh0, ow0, thn, twn);
      }
      return;
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
  if (p.hist) tile_halo_hist(p, off_l, p.GW, oh0, ow0, thn, twn);

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
// Direct-gather variant: the corners are read straight from a channel-minor
// copy of the input (one 16-byte load = 8 bf16 or 4 fp32 channels of one
// corner), which stays resident in the L2s and the 256 MB Infinity Cache; no
// input staging, no halo, no chunk loop and no barriers in the blend.  The
// offset conv reads its MFMA operand fragments from the same copy.  Out-of-
// image corners read the copy's extra zero pixel, so fully outside taps blend
// to zero without a special case.
// MODE: kFusedMode (offset conv + sampling), kOffsetsMode (offset conv only,
// offsets to off_out), kSampleMode (sampling from offsets read from off_in).
template <typename T, int MB, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_sample_direct(const SampleParams p) {
  constexpr int VEC = Elem<T>::VEC, ESZ = (int)sizeof(T);
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lw = xcd_swizzle(blockIdx.x, p.num_wg);
  const int tile = lw / p.gsplit, gs = lw - tile * p.gsplit;
  const int tpi = p.tiles_h * p.tiles_w;
  const int n = tile / tpi, trem = tile - n * tpi;
  const int tyi = trem / p.tiles_w, txi = trem - tyi * p.tiles_w;
  const int oh0 = tyi * p.TH, ow0 = txi * p.TW;
  const int thn = min(p.TH, p.Ho - oh0), twn = min(p.TW, p.Wo - ow0);
  const int PT = p.TH * p.TW;
  const int g = gs;  // one offset group per workgroup
  const int ocw = 2 * p.K2;
  const int obase = 2 * g * p.K2;
  const int HW = p.H * p.W;
  float* off_l = (float*)(smem + p.lds_off);                                  // [ocw][PT]
  int4* tab = (int4*)(smem + p.lds_info);                                     // [PT][K2] corner byte offsets
  float4* wts = (float4*)(smem + p.lds_info + PT * p.K2 * 16);                // [PT][K2] corner weights
  int* cof = (int*)(smem + p.lds_info + PT * p.K2 * 32);                      // [PT][K2] column offset
  const T* __restrict__ xn = (const T*)p.xh + (size_t)n * (HW + 1) * p.Cin;
  const int fy0 = oh0 * p.SH - p.PH, fx0 = ow0 * p.SW - p.PW;

  if constexpr (MODE == kSampleMode) {
    // offsets of this tile from global memory (the unfused formulation)
    const int tot = ocw * PT;
    for (int e = tid; e < tot; e += 256) {
      const int o = e / PT, pix = e - o * PT;
      const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
      float v = 0.f;
      if (ty < thn && tx < twn)
        v = p.off_in[(((size_t)n * p.Oc + obase + o) * p.Ho + oh0 + ty) * p.Wo + ow0 + tx];
      off_l[e] = v;
    }
    __syncthreads();
  } else {
  // ---- phase A: offsets of this tile, operand fragments from the copy ----
    // The offset-conv bias of this thread's elements of the reduction below
    // (at most four: e = tid + 256 k < ocw * PT <= 1152), loaded now so the
    // reduction does not wait on them.
    const int tot = ocw * PT;
    float bias4[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int e = tid + 256 * k;
      bias4[k] = p.b_off && e < tot ? Elem<T>::to_f32(((const T*)p.b_off)[obase + e / PT]) : 0.f;
    }
    f32x16_t acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;
    // Same unit walk as the LDS-staged kernel (bit-identical offsets); a
    // unit here is one batch (at most four k-steps: CA <= 64 bf16 or 32 fp32
    // channels).  The
    // tile's footprint, one chunk of CA channels at a time, is copied from
    // the channel-minor input into LDS by direct buffer-to-LDS loads (whole
    // 16-byte pieces of contiguous pixel rows), double buffered; 16-byte
    // piece q of footprint pixel P sits in slot P * nq + (q ^ (P % nq)), so
    // the 32 pixels of an operand read hit distinct banks.  The weights come
    // in fragment order: one 1 KB contiguous load per k-step.
    const int nks = p.CA / (2 * VEC), nch = p.Cin / p.CA, nq = p.CA / VEC;
    const int nslot = p.FH * p.FW * nq;
    const int D = p.stage_d;
    unsigned char* stg = smem + p.lds_region;  // [2][D * 256 slots][16 B]
    const rsrc_t xr = make_rsrc(xn, (uint32_t)((size_t)(HW + 1) * p.Cin * ESZ));
    const bool nb1 = PT > 32;
    const T* __restrict__ wf = (const T*)p.woff_p + (size_t)g * p.K2 * p.Cin * 32 + lane * VEC;
    int pixb[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      int pix = nb * 32 + (lane & 31);
      if (pix >= PT) pix = 0;
      const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
      pixb[nb] = ty * p.SH * p.FW + tx * p.SW;  // footprint pixel of tap (0,0)
    }
    auto issue = [&](int c, int buf) {
      unsigned char* b = stg + buf * (D * 4096);
      for (int i = 0; i < D; ++i) {
        const int s0 = (i * 4 + wave) * 64, sl = s0 + lane;
        int voff = kOOB;
        if (sl < nslot) {
          const int P = sl / nq, q = (sl - P * nq) ^ (P & (nq - 1));
          const int fy = fdiv(P, p.div_fw), fx = P - fy * p.FW;
          const int y = fy0 + fy, xx = fx0 + fx;
          const int pix = ((unsigned)y < (unsigned)p.H && (unsigned)xx < (unsigned)p.W) ? y * p.W + xx : HW;
          voff = (pix * p.Cin + c * p.CA + q * VEC) * ESZ;
        }
        load_lds16(xr, b + s0 * 16, voff);
      }
    };
    // Weights of this wave's units of one chunk (at most three: K2 <= 9);
    // unit u of chunk c + 1 is loaded into wa[u] as soon as unit u of chunk
    // c has been multiplied, so its latency hides behind the rest.
    uint4 wa[3][4];
    int tl[3], nu = 0;
    UnitWalk uw;
    uw.start(wave, p.K2);
    auto fetch = [&](int c) {  // walks uw over chunk c's units, loading their weights
      nu = 0;
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        if (uw.c == c) {
          tl[u] = uw.t; nu = u + 1;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (k < nks) wa[u][k] = *(const uint4*)(wf + ((size_t)(uw.t * nch + c) * nks + k) * (64 * VEC));
          uw.next(p.K2, nks);
        }
      }
    };
    issue(0, 0);
    fetch(0);
    for (int c = 0; c < nch; ++c) {
      wait_vm<0>();     // this wave's pieces of chunk c and its weights have landed
      __syncthreads();  // everyone's have; everyone is done with chunk c - 1
      if (c + 1 < nch) issue(c + 1, (c + 1) & 1);
      const unsigned char* b = stg + (c & 1) * (D * 4096);
      const int nuc = nu;
      int tlc[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) tlc[u] = tl[u];
      // next chunk's units (same count pattern; loaded per unit below);
      // none after the last chunk
      UnitWalk un = uw;
      int tn[3], nn = 0;
#pragma unroll
      for (int u = 0; u < 3; ++u)
        if (un.c == c + 1 && c + 1 < nch) { tn[u] = un.t; nn = u + 1; un.next(p.K2, nks); }
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        if (u < nuc) {
          const int ti = tlc[u] / p.KW, tj = tlc[u] - ti * p.KW;
          const int toff = ti * p.DH * p.FW + tj * p.DW;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (k >= nks) break;
            const int q = (lane >> 5) * (nq >> 1) + k;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
              if (nb == 1 && !nb1) break;
              const int P = pixb[nb] + toff;
              const uint4 bq = *(const uint4*)(b + (P * nq + (q ^ (P & (nq - 1)))) * 16);
              mfma_chunk(acc[0][nb], wa[u][k], bq, T());
            }
          }
        }
        if (u < nn) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (k < nks) wa[u][k] = *(const uint4*)(wf + ((size_t)(tn[u] * nch + c + 1) * nks + k) * (64 * VEC));
        }
      }
#pragma unroll
      for (int u = 0; u < 3; ++u) tl[u] = tn[u];
      nu = nn;
      uw = un;
    }
    __syncthreads();  // the partial sums below reuse the staging buffers
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
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int e = tid + 256 * k;
      if (e >= tot) break;
      const int o = e / PT, pix = e - o * PT;
      float v = part[e] + part[tot + e];
      v += part[2 * tot + e];
      v += part[3 * tot + e];
      v += bias4[k];
      off_l[e] = v;
      const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
      if (p.off_out && ty < thn && tx < twn)
        p.off_out[(((size_t)n * p.Oc + obase + o) * p.Ho + oh0 + ty) * p.Wo + ow0 + tx] = v;
    }
    if constexpr (MODE == kOffsetsMode) {
      // the offsets alone (the gather-fused forward samples in its GEMM);
      // their histogram still counts
      if (p.hist) {
        __syncthreads();
        tile_halo_hist(p, off_l, 1, oh0, ow0, thn, twn);
      }
      return;
    }
    __syncthreads();
  }

  if (p.hist) tile_halo_hist(p, off_l, 1, oh0, ow0, thn, twn);
  // ---- tap index stage: corner byte offsets, column offset, weights ----
  // A corner outside the image (and every corner of a fully outside tap)
  // points at the copy's zero pixel; -1 marks a pixel beyond the tile.
  const int nent = PT * p.K2;
  const int zpix = HW * p.Cin * ESZ;
  for (int e = tid; e < nent; e += 256) {
    const int pix = fdiv(e, p.div_k2), t = e - pix * p.K2;
    const int ty = fdiv(pix, p.div_tw), tx = pix - ty * p.TW;
    int4 tb = make_int4(zpix, zpix, zpix, zpix);
    int co = -1;
    float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ty < thn && tx < twn) {
      const int ti = t / p.KW, tj = t - ti * p.KW;
      const int by = (oh0 + ty) * p.SH - p.PH + ti * p.DH;
      const int bx = (ow0 + tx) * p.SW - p.PW + tj * p.DW;
      const float dy = off_l[(2 * t) * PT + pix];
      const float dx = off_l[(2 * t + 1) * PT + pix];
      const TapIndex ix = tap_index(by, bx, dy, dx, p.H, p.W);
      co = (ty * p.Wo + tx) * p.Ck + t * p.Cin;
      if (!ix.outside) {
        const int b = (ix.y0 * p.W + ix.x0) * p.Cin * ESZ, cw1 = p.Cin * ESZ, cwW = p.W * p.Cin * ESZ;
        const uint32_t m = corner_mask(ix, p.H, p.W);
        tb.x = (m & 1) ? b : zpix;
        tb.y = (m & 2) ? b + cw1 : zpix;
        tb.z = (m & 4) ? b + cwW : zpix;
        tb.w = (m & 8) ? b + cwW + cw1 : zpix;
        float w[4];
        tap_weights(ix, w);
        wv = make_float4(w[0], w[1], w[2], w[3]);
      }
    }
    tab[e] = tb;
    wts[e] = wv;
    cof[e] = co;
  }
  __syncthreads();

  // ---- phase B: every (pixel, tap) x 16 bytes of channels, corners from the copy ----
  // 32-bit buffer offsets: the table's corner offset plus the lane's channels.
  const int nvm = (1 << p.nv_log) - 1;
  const int v = tid & nvm, e0 = tid >> p.nv_log, estep = 256 >> p.nv_log;
  const int cofs = g * p.Cg + v * VEC;
  const __amdgpu_buffer_rsrc_t xb = make_brsrc(xn, (uint32_t)((size_t)(HW + 1) * p.Cin * ESZ));
  const int lofs = cofs * ESZ;
  T* __restrict__ colt = (T*)p.cols + ((size_t)n * p.Ho * p.Wo + (size_t)oh0 * p.Wo + ow0) * p.Ck + cofs;
  for (int e = e0; e < nent; e += 2 * estep) {
    int co[2];
    float w[2][4];
    uint4 q[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int eu = e + u * estep;
      const int ec = eu < nent ? eu : e;
      const int4 tb = tab[ec];
      co[u] = eu < nent ? cof[ec] : -1;
      const float4 wq = wts[ec];
      w[u][0] = wq.x; w[u][1] = wq.y; w[u][2] = wq.z; w[u][3] = wq.w;
      q[u][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xb, tb.x + lofs, 0, 0));
      q[u][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xb, tb.y + lofs, 0, 0));
      q[u][2] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xb, tb.z + lofs, 0, 0));
      q[u][3] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xb, tb.w + lofs, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (co[u] < 0) continue;
      if constexpr (VEC == 8) {
        float f00[8], f01[8], f10[8], f11[8], o8[8];
        unpack8(q[u][0], f00);
        unpack8(q[u][1], f01);
        unpack8(q[u][2], f10);
        unpack8(q[u][3], f11);
#pragma unroll
        for (int c = 0; c < 8; ++c) o8[c] = blend4(w[u], f00[c], f01[c], f10[c], f11[c]);
        store8_nt((bf16_t*)(colt + co[u]), o8);
      } else {
        auto bl = [&](uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
          return __float_as_uint(
              blend4(w[u], __uint_as_float(a), __uint_as_float(b), __uint_as_float(c), __uint_as_float(d)));
        };
        const uint4 o4 = make_uint4(bl(q[u][0].x, q[u][1].x, q[u][2].x, q[u][3].x),
                                    bl(q[u][0].y, q[u][1].y, q[u][2].y, q[u][3].y),
                                    bl(q[u][0].z, q[u][1].z, q[u][2].z, q[u][3].z),
                                    bl(q[u][0].w, q[u][1].w, q[u][2].w, q[u][3].w));
        store16_nt(colt + co[u], o4);
      }
    }
  }
}

// x [N][Cin][H*W] -> xh [N][H*W+1][Cin] (bf16), pixel H*W of every image zero.
// Each lane moves an 8 x 8 block (8 channels x 8 pixels): eight 16-byte loads
// along the pixels, a register transpose with byte permutes, eight 16-byte
// stores along the channels.  A wave covers 64 pixels x 64 channels, so both
// the loads and the stores come in whole 128-byte runs.
__device__ __forceinline__ void x_channel_minor_body(int bid, const bf16_t* __restrict__ x, bf16_t* __restrict__ xh,
                                                     int Cin, int HW, int pgroups, int cgroups, int total_waves) {
  const int lane = threadIdx.x & 63;
  const int wv = bid * 4 + (threadIdx.x >> 6);
  if (wv >= total_waves) return;
  const int cgi = wv % cgroups, r = wv / cgroups;
  const int pgi = r % pgroups, n = r / pgroups;
  const int c = cgi * 64 + (lane & 7) * 8;
  const int p0 = pgi * 64 + (lane >> 3) * 8;
  if (c >= Cin || p0 > HW) return;
  const bf16_t* src = x + ((size_t)n * Cin + c) * HW;
  uint4 rv[8];
  if ((HW & 7) == 0 && p0 + 8 <= HW) {
#pragma unroll
    for (int k = 0; k < 8; ++k) rv[k] = *(const uint4*)(src + (size_t)k * HW + p0);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = p0 + i < HW ? (uint32_t)src[(size_t)k * HW + p0 + i] : 0u;
      rv[k] = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16);
    }
  }
  bf16_t* dst = xh + ((size_t)n * (HW + 1) + p0) * Cin + c;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // pixel i sits in dword i/2 of every channel's word, low half for even i
    const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
    auto dw = [&](const uint4& q) { return (i >> 1) == 0 ? q.x : (i >> 1) == 1 ? q.y : (i >> 1) == 2 ? q.z : q.w; };
    uint4 o;
    o.x = __builtin_amdgcn_perm(dw(rv[1]), dw(rv[0]), sel);
    o.y = __builtin_amdgcn_perm(dw(rv[3]), dw(rv[2]), sel);
    o.z = __builtin_amdgcn_perm(dw(rv[5]), dw(rv[4]), sel);
    o.w = __builtin_amdgcn_perm(dw(rv[7]), dw(rv[6]), sel);
    if (p0 + i <= HW) *(uint4*)(dst + (size_t)i * Cin) = o;
  }
}

// fp32: x [N][Cin][H*W] -> xh [N][H*W+1][Cin], pixel H*W of every image
// zero.  One workgroup moves a 64-channel x 64-pixel tile through LDS: loads
// of 16 consecutive pixels x 4 per lane group (256-byte runs along the
// pixels), stores of 16 channel quads (256-byte runs along the channels); the
// LDS rows hold 65 floats, so both the scalar writes and the transposed
// reads hit 64 distinct banks.
__global__ __launch_bounds__(256) void k_x_channel_minor_f32(const float* __restrict__ x, float* __restrict__ xh,
                                                             int Cin, int HW, int pblocks, int cblocks) {
  __shared__ float tl[64 * 65];
  const int t = threadIdx.x;
  const int b = blockIdx.x;
  const int cb = b % cblocks, r = b / cblocks;
  const int pb = r % pblocks, n = r / pblocks;
  const int c0 = cb * 64, p0 = pb * 64;
  const float* src = x + (size_t)n * Cin * HW;
  const bool vec = (HW & 3) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ci = (t >> 4) + 16 * i, pq = (t & 15) * 4;
    const int c = c0 + ci, p = p0 + pq;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < Cin) {
      const float* row = src + (size_t)c * HW;
      if (vec && p + 4 <= HW) {
        v = *(const float4*)(row + p);
      } else {
        v.x = p < HW ? row[p] : 0.f;
        v.y = p + 1 < HW ? row[p + 1] : 0.f;
        v.z = p + 2 < HW ? row[p + 2] : 0.f;
        v.w = p + 3 < HW ? row[p + 3] : 0.f;
      }
    }
    tl[ci * 65 + pq] = v.x;
    tl[ci * 65 + pq + 1] = v.y;
    tl[ci * 65 + pq + 2] = v.z;
    tl[ci * 65 + pq + 3] = v.w;
  }
  __syncthreads();
  float* dst = xh + (size_t)n * (HW + 1) * Cin;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pi = (t >> 4) + 16 * i, cq = (t & 15) * 4;
    const int p = p0 + pi, c = c0 + cq;
    if (p > HW || c >= Cin) continue;
    const float4 v = make_float4(tl[cq * 65 + pi], tl[(cq + 1) * 65 + pi], tl[(cq + 2) * 65 + pi], tl[(cq + 3) * 65 + pi]);
    *(float4*)(dst + (size_t)p * Cin + c) = v;
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
// Weights of the main conv -> Wt [Cout][taps][Cin]; offset-conv weights ->
// rows [OcP][taps][Cin] (LDS-staged sampling kernel), or with CA > 0 the
// direct kernel's fragment order: per group, tap, chunk of CA channels and
// k-step, the 64 lanes' 16-byte A operands back to back (lane L: offset
// channel L % 32 of the group, zero past 2 * taps; channels
// chunk * CA + (L / 32) * CA / 2 + step * V ... + V - 1, V = 8 bf16 or 4
// fp32 elements per 16 bytes).
template <typename T>
__device__ __forceinline__ void prep_forward_body(int bid, int nblocks, const T* __restrict__ w,
                                                  const T* __restrict__ w_off, T* wt, T* woff_p, int Cout, int Cin,
                                                  int K2, int Oc, int OcP, int G, int CA) {
  const size_t n1 = (size_t)Cout * K2 * Cin;
  const size_t n2 = CA > 0 ? (size_t)G * K2 * Cin * 32 : (size_t)OcP * K2 * Cin;
  constexpr int V = Elem<T>::VEC, LV = V == 8 ? 3 : 2;
  const int nks = CA / (2 * V), nch = CA > 0 ? Cin / CA : 1;
  for (size_t e = (size_t)bid * 256 + threadIdx.x; e < n1 + n2; e += (size_t)nblocks * 256) {
    // weight tensors are far below 2^31 elements: 32-bit index arithmetic
    if (e < n1) {
      const int ei = (int)e;
      const int r = ei / Cin, c = ei - r * Cin;
      const int co = r / K2, t = r - co * K2;
      wt[e] = w[(co * Cin + c) * K2 + t];
    } else if (CA > 0) {
      const int f = (int)(e - n1);
      const int e8 = f & (V - 1), L = (f >> LV) & 63;
      int r = f >> (LV + 6);
      const int k = r % nks; r /= nks;
      const int ch = r % nch; r /= nch;
      const int t = r % K2;
      const int g = r / K2;
      const int ol = L & 31;
      const int c = ch * CA + (L >> 5) * (CA / 2) + k * V + e8;
      woff_p[f] = ol < 2 * K2 ? w_off[((2 * g * K2 + ol) * Cin + c) * K2 + t] : zero_elem<T>();
    } else {
      const int f = (int)(e - n1);
      const int r = f / Cin, c = f - r * Cin;
      const int o = r / K2, t = r - o * K2;
      woff_p[f] = o < Oc ? w_off[(o * Cin + c) * K2 + t] : zero_elem<T>();
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_prep_forward(const T* __restrict__ w, const T* __restrict__ w_off,
                                                      T* wt, T* woff_p, int Cout, int Cin, int K2, int Oc,
                                                      int OcP, int G, int CA) {
  prep_forward_body<T>(blockIdx.x, gridDim.x, w, w_off, wt, woff_p, Cout, Cin, K2, Oc, OcP, G, CA);
}

// The direct-gather forward's prologue in one launch: the first nxb
// workgroups build the channel-minor copy of x, the rest lay out the weights.
__global__ __launch_bounds__(256) void k_x_channel_minor_prep(const bf16_t* __restrict__ x, bf16_t* __restrict__ xh,
                                                              int Cin, int HW, int pgroups, int cgroups,
                                                              int total_waves, int nxb, const bf16_t* __restrict__ w,
                                                              const bf16_t* __restrict__ w_off, bf16_t* wt,
                                                              bf16_t* woff_p, int Cout, int K2, int Oc, int OcP, int G,
                                                              int CA) {
  if ((int)blockIdx.x < nxb)
    x_channel_minor_body(blockIdx.x, x, xh, Cin, HW, pgroups, cgroups, total_waves);
  else
    prep_forward_body<bf16_t>(blockIdx.x - nxb, gridDim.x - nxb, w, w_off, wt, woff_p, Cout, Cin, K2, Oc, OcP, G,
                              CA);
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
  s.div_fw = make_fastdiv(p.foot_w);
  s.stage_d = p.stage_d;
  s.xh = nullptr;
  s.nv_log = 0;
  s.offsets_only = 0;
  s.hist = a.hist;
  s.hist_len = a.hist_len;
  s.x = a.x; s.woff_p = a.woff_p; s.b_off = a.b_off; s.off_in = a.off_in; s.off_out = a.off_out;
  s.cols = a.cols;
  return s;
}

template <typename T, bool FUSED, int MB>
static hipError_t launch_sample_t(const deft_plan& p, const SampleParams& s, const char* name, hipStream_t st) {
  auto kern = k_sample<T, FUSED, MB>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_total);
  if (e != hipSuccess) return e;
  DEFT_LAUNCH(name, kern, dim3(p.num_wg), dim3(256), p.lds_total, st, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_sample_dt(const deft_plan& p, SampleMode mode, const SampleParams& s, hipStream_t st) {
  if (mode == kSampleMode) return launch_sample_t<T, false, 1>(p, s, "sample_only", st);
  const char* name = mode == kOffsetsMode ? "offset_conv" : "fused_offset_sample";
  switch (p.mblocks) {
    case 1: return launch_sample_t<T, true, 1>(p, s, name, st);
    case 2: return launch_sample_t<T, true, 2>(p, s, name, st);
    case 3: return launch_sample_t<T, true, 3>(p, s, name, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int MODE>
static hipError_t launch_direct_t(const deft_plan& p, const SampleParams& s, const char* name, hipStream_t st) {
  auto kern = k_sample_direct<T, 1, MODE>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_total);
  if (e != hipSuccess) return e;
  DEFT_LAUNCH(name, kern, dim3(p.num_wg), dim3(256), p.lds_total, st, s);
  return hipGetLastError();
}

hipError_t launch_sample(const deft_plan& p, SampleMode mode, const SampleArgs& a, hipStream_t st) {
  SampleParams s = make_params(p, a);
  s.offsets_only = mode == kOffsetsMode;
  if (p.num_wg == 0) return hipSuccess;
  if (p.direct && a.xh) {
    // the gather from the channel-minor copy (built by the prologue launch)
    s.xh = a.xh;
    const bool bf = p.d.dtype == DEFT_BF16;
    int l = 0;
    while ((1 << l) < p.cg / (bf ? 8 : 4)) ++l;
    s.nv_log = l;
    if (p.mblocks != 1) return hipErrorInvalidValue;
    switch (mode) {
      case kFusedMode:
        return bf ? launch_direct_t<bf16_t, kFusedMode>(p, s, "fused_offset_sample", st)
                  : launch_direct_t<float, kFusedMode>(p, s, "fused_offset_sample", st);
      case kOffsetsMode:
        return bf ? launch_direct_t<bf16_t, kOffsetsMode>(p, s, "offset_conv", st)
                  : launch_direct_t<float, kOffsetsMode>(p, s, "offset_conv", st);
      default:
        return bf ? launch_direct_t<bf16_t, kSampleMode>(p, s, "sample_only", st)
                  : launch_direct_t<float, kSampleMode>(p, s, "sample_only", st);
    }
  }
  return p.d.dtype == DEFT_BF16 ? launch_sample_dt<bf16_t>(p, mode, s, st)
                                : launch_sample_dt<float>(p, mode, s, st);
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
                               void* woff_p, const void* x, void* xh, hipStream_t st) {
  const deft_desc& d = p.d;
  const int ca = p.direct ? p.chunk_a : 0;
  const size_t total = (size_t)d.c_out * p.taps * d.c_in +
                       (ca ? (size_t)d.offset_groups * p.taps * d.c_in * 32 : (size_t)p.oc_pad * p.taps * d.c_in);
  unsigned g = grid_for(total);
  if (g > 4096) g = 4096;
  if (p.direct && d.dtype != DEFT_BF16) {
    // fp32: the channel-minor copy, then the weights (offset conv in fragment order)
    const int HW = d.h * d.w;
    const int pblocks = (HW + 1 + 63) / 64, cblocks = (d.c_in + 63) / 64;
    DEFT_LAUNCH("x_channel_minor", k_x_channel_minor_f32, dim3(d.n * pblocks * cblocks), dim3(256), 0, st,
                (const float*)x, (float*)xh, d.c_in, HW, pblocks, cblocks);
    DEFT_LAUNCH("prep_forward", k_prep_forward<float>, dim3(g), dim3(256), 0, st, (const float*)w,
                (const float*)w_off, (float*)wt, (float*)woff_p, d.c_out, d.c_in, p.taps, p.oc, p.oc_pad,
                d.offset_groups, ca);
    return hipGetLastError();
  }
  if (p.direct) {
    const int HW = d.h * d.w;
    const int pgroups = (HW + 1 + 63) / 64, cgroups = (d.c_in + 63) / 64;
    const int waves = d.n * pgroups * cgroups, nxb = (waves + 3) / 4;
    DEFT_LAUNCH("x_channel_minor", k_x_channel_minor_prep, dim3(nxb + g), dim3(256), 0, st, (const bf16_t*)x,
                (bf16_t*)xh, d.c_in, HW, pgroups, cgroups, waves, nxb, (const bf16_t*)w, (const bf16_t*)w_off,
                (bf16_t*)wt, (bf16_t*)woff_p, d.c_out, p.taps, p.oc, p.oc_pad, d.offset_groups, ca);
    return hipGetLastError();
  }
  if (d.dtype == DEFT_BF16)
    DEFT_LAUNCH("prep_forward", k_prep_forward<bf16_t>, dim3(g), dim3(256), 0, st, (const bf16_t*)w,
                       (const bf16_t*)w_off, (bf16_t*)wt, (bf16_t*)woff_p, d.c_out, d.c_in, p.taps, p.oc,
                       p.oc_pad, d.offset_groups, ca);
  else
    DEFT_LAUNCH("prep_forward", k_prep_forward<float>, dim3(g), dim3(256), 0, st, (const float*)w,
                       (const float*)w_off, (float*)wt, (float*)woff_p, d.c_out, d.c_in, p.taps, p.oc,
                       p.oc_pad, d.offset_groups, ca);
  return hipGetLastError();
}

}  // namespace deft
