// C ABI of the deformable convolution library: descriptor validation, the
// tile planner, workspace layout and launch sequencing.  Everything here runs
// on the host; kernels live in deft_sample.hip, deft_gemm.hip and
// deft_backward.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "deft.h"
#include "deft_internal.h"

namespace {

thread_local char g_last_hip[256] = "";

int hip_fail(hipError_t e) {
  std::snprintf(g_last_hip, sizeof(g_last_hip), "%s (%d)", hipGetErrorString(e), (int)e);
  return DEFT_ERR_HIP;
}

// Compute units and LDS bytes per workgroup of the current device, read once
// per device; without a device (planning on a host with no GPU) those of
// MI355X: 256 CUs, 160 KB.
struct DeviceLimits {
  int cus = 256, max_lds = 160 * 1024;
};
DeviceLimits device_limits() {
  static DeviceLimits cache[64];
  static bool known[64] = {false};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return DeviceLimits{};
  }
  if (!known[dev]) {
    DeviceLimits l;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) l.cus = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
      l.max_lds = v;
    (void)hipGetLastError();
    cache[dev] = l;
    known[dev] = true;
  }
  return cache[dev];
}

// A plan for descriptor d on the current device (fields not yet laid out).
deft_plan blank_plan(const deft_desc& d, const DeviceLimits& lim) {
  deft_plan p;
  p.d = d;
  p.cus = lim.cus;
  p.max_lds = lim.max_lds;
  return p;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
int align16(int v) { return (v + 15) & ~15; }

int out_dim(int in, int k, int s, int p, int d) { return (in + 2 * p - d * (k - 1) - 1) / s + 1; }

int validate(const deft_desc* d) {
  if (!d) return DEFT_ERR_NULLPTR;
  if (d->dtype != DEFT_F32 && d->dtype != DEFT_BF16) return DEFT_ERR_DTYPE;
  if (d->n < 0 || d->c_in < 1 || d->h < 1 || d->w < 1 || d->c_out < 1 || d->kh < 1 || d->kw < 1 ||
      d->stride_h < 1 || d->stride_w < 1 || d->dil_h < 1 || d->dil_w < 1 || d->pad_h < 0 || d->pad_w < 0)
    return DEFT_ERR_BAD_DESC;
  if (d->offset_groups < 1 || d->c_in % d->offset_groups != 0) return DEFT_ERR_GROUPS;
  if (out_dim(d->h, d->kh, d->stride_h, d->pad_h, d->dil_h) < 1 ||
      out_dim(d->w, d->kw, d->stride_w, d->pad_w, d->dil_w) < 1)
    return DEFT_ERR_SHAPE;
  if ((d->c_in / d->offset_groups) % 16 != 0) return DEFT_ERR_UNSUPPORTED;
  if (d->h >= 32767 || d->w >= 32767 || d->kh * d->kw > 48) return DEFT_ERR_UNSUPPORTED;
  const double x_elems = (double)d->n * d->c_in * d->h * d->w;
  const double col_elems = (double)d->n * out_dim(d->h, d->kh, d->stride_h, d->pad_h, d->dil_h) *
                           out_dim(d->w, d->kw, d->stride_w, d->pad_w, d->dil_w) * d->c_in * d->kh * d->kw;
  const double pairs = col_elems / (d->c_in * d->kh * d->kw) * d->offset_groups * d->kh * d->kw;
  if (x_elems >= 2147483647.0 || (double)d->n * d->c_out * d->h * d->w >= 2147483647.0 ||
      col_elems / (d->c_in * d->kh * d->kw) >= 2147483647.0 || pairs >= 2147483647.0 ||
      (double)(d->c_out + 2.0 * d->offset_groups * d->kh * d->kw + 64) * d->c_in * d->kh * d->kw >= 2147483647.0)
    return DEFT_ERR_UNSUPPORTED;
  return DEFT_OK;
}

struct Shape {
  int ho, wo, taps, oc, cg, ck, esz;
};
Shape shape_of(const deft_desc& d) {
  Shape s;
  s.ho = out_dim(d.h, d.kh, d.stride_h, d.pad_h, d.dil_h);
  s.wo = out_dim(d.w, d.kw, d.stride_w, d.pad_w, d.dil_w);
  s.taps = d.kh * d.kw;
  s.oc = 2 * d.offset_groups * s.taps;
  s.cg = d.c_in / d.offset_groups;
  s.ck = d.c_in * s.taps;
  s.esz = d.dtype == DEFT_BF16 ? 2 : 4;
  return s;
}

// Backward tiling: the sampling backward gives each workgroup a core tile of
// input pixels; the (output pixel, tap) pairs whose corners touch the core
// (within the halo) are gathered into a list, then per channel chunk dCol x
// weight is summed into the core (bf16: as MFMA products of weight tiles with
// the staged dCol rows; fp32: in a fixed-point LDS copy of the core, lanes =
// channels) and the core's dX is written once.  A pair straddling two cores is read by both, so
// larger cores read dCol fewer times; the LDS holds the core plus a one-pixel
// ring of the input (for the offset gradient) and the fp32 core.
bool layout_backward(deft_plan& p) {
  const deft_desc& d = p.d;
  const Shape s = shape_of(d);
  // 8x8 cores keep several workgroups per CU; chunk = 64 channels (one per
  // lane) when the group allows it
  const int ch = std::min(8, d.h), cw = std::min(8, d.w);
  int cb = 64;
  while (cb > 16 && s.cg % cb) cb /= 2;
  if (s.cg % cb) return false;
  const int vec = d.dtype == DEFT_BF16 ? 8 : 4;
  // bf16 with a core of at most 64 pixels and 32 or 64 channels: the scatter
  // runs on the MFMA units (its buffer offsets into one image's dCol rows
  // are 32-bit)
  const bool mf = d.dtype == DEFT_BF16 && ch * cw <= 64 && cb % 32 == 0 &&
                  (size_t)s.ho * s.wo * s.ck * 2 < ((size_t)1 << 31);
  const int xstr = mf ? cb : cb + vec;  // staged input pixel stride (elements)
  const int lx = align16((ch + 2) * (cw + 2) * xstr * s.esz);
  int ldx, ldc, lfl = 0;
  if (mf) {
    // blocks of blk = 2048 / cb list entries: two buffers of bf16 weight
    // tiles (hi and lo, [64 pixels][blk]), two staged dCol tiles [blk][cb],
    // 4-bit non-finite flags per (pixel, channel) and one word
    const int blk = 2048 / cb;
    ldx = 2 * 2 * 64 * blk * 2;
    ldc = 2 * blk * cb * 2;
    lfl = 64 * cb / 2 + 16;
  } else {
    // fixed-point dX of the core, spill slots, non-finite flags (4 bits per element)
    ldx = align16((ch * cw * cb + 64) * (d.dtype == DEFT_BF16 ? 4 : 8) + (ch * cw * cb + 7) / 8 * 4);
    ldc = 4 * 32 * (cb + vec) * s.esz;  // 4 waves x 32 rows
  }
  const int total = lx + ldx + ldc + lfl;
  if (total > p.max_lds) return false;
  p.btile_h = ch; p.btile_w = cw;
  p.btiles_h = (d.h + ch - 1) / ch; p.btiles_w = (d.w + cw - 1) / cw;
  p.num_btiles = d.n * p.btiles_h * p.btiles_w;
  p.chunk_b = cb;
  p.bwd_mf = mf ? 1 : 0;
  p.lb_dx = lx; p.lb_dc = lx + ldx; p.lb_cnt = lx + ldx + ldc; p.lb_total = total;
  // list capacity: every output pixel whose tap's grid point lies within the
  // halo (plus one row/column for the +1 corners) of the core, for every tap
  const int wh = (p.btile_h + 2 * p.bhalo + 1 + d.stride_h - 1) / d.stride_h + 1;
  const int ww = (p.btile_w + 2 * p.bhalo + 1 + d.stride_w - 1) / d.stride_w + 1;
  p.list_cap = s.taps * std::min(wh, s.ho) * std::min(ww, s.wo);
  // offset-weight backward: (image, channel slice, row band) workgroups, four
  // per CU in the bf16-operand form, else two (one where a launch covers
  // more than 32 offset channels); a band's input rows are staged at once.
  // The band count minimises an estimate of the launch plus the reduction of
  // its partials: the staged rows per workgroup times the rounds of
  // workgroups (fractional past the first), plus the partials' bytes at about
  // 4.5 TB/s, counted in the same unit (a staged row takes about 2.8 us per
  // round); the fewest bands among equals.
  const int slices = (d.c_in + 31) / 32;
  const int kc = d.dtype == DEFT_BF16 ? 16 : 8;
  const int wop = (s.wo + kc - 1) / kc * kc;
  const int span = (wop - 1) * d.stride_w + (d.kw - 1) * d.dil_w + 1;
  const int xs = ((8 + span + 7) / 8) * 8;  // bound on the staged row length
  const int mbw = std::min(3, (s.oc + 31) / 32);
  auto woff_lds = [&](int rows) {
    const int xr = (rows - 1) * d.stride_h + (d.kh - 1) * d.dil_h + 1;
    // bf16 reads its dOffset operand from global memory; fp32 stages it too
    return align16(32 * xr * xs * s.esz) + (d.dtype == DEFT_BF16 ? 0 : mbw * 32 * rows * (wop + vec) * s.esz);
  };
  const int per_cu = deft::woff_a16(d.dtype, s.oc, s.wo) ? 4 : (mbw == 1 ? 2 : 1);
  const long slots = (long)std::max(1, p.cus) * per_cu;
  int bands = 0;
  double best = 0.0;
  for (int nb = 1; nb <= s.ho; ++nb) {
    const int rows = (s.ho + nb - 1) / nb;
    if (woff_lds(rows) > p.max_lds / std::max(2, per_cu)) continue;
    const double rounds = std::max(1.0, (double)d.n * slices * nb / (double)slots);
    const double partials = (double)d.n * nb * s.oc * s.ck * 4;
    const double cost = rounds * ((rows - 1) * d.stride_h + (d.kh - 1) * d.dil_h + 1) + partials / 12.6e6;
    if (!bands || cost < best - 1e-9) { bands = nb; best = cost; }
  }
  if (!bands) bands = s.ho;
  // the offset-weight backward stages whole input rows: a band of the rows
  // it settled on must fit the LDS, else this shape has no backward here
  if (woff_lds((s.ho + bands - 1) / bands) > p.max_lds) return false;
  p.woff_bands = bands;
  return true;
}

// The direct-gather forward (corners from a channel-minor copy of x) needs
// at most 9 taps (one block of offset channels, at most three units per wave
// and chunk), a power-of-two number of 16-byte channel slices per group (8
// bf16 or 4 fp32 channels; at most 256) and byte offsets below 2^31 within
// one image's copy.
bool direct_ok(const deft_desc& d) {
  const Shape s = shape_of(d);
  const int vec = d.dtype == DEFT_BF16 ? 8 : 4;
  const int nv = s.cg / vec;
  return d.c_in % 16 == 0 && s.cg % vec == 0 && s.taps <= 9 && nv >= 1 && nv <= 256 && (nv & (nv - 1)) == 0 &&
         ((size_t)d.h * d.w + 1) * d.c_in * (d.dtype == DEFT_BF16 ? 2 : 4) < 0x80000000u;
}

// Fills every derived field of a plan for the given tile / halo / chunk
// (direct: the forward gathers from the channel-minor copy and has no LDS
// halo) and the backward's halo (negative: the forward's).  Returns false
// if the LDS does not fit.
bool layout_plan(deft_plan& p, int th, int tw, int halo, int chunk, bool direct = false, int bhalo = -1) {
  const deft_desc& d = p.d;
  const Shape s = shape_of(d);
  if (direct && !direct_ok(d)) return false;
  p.direct = direct ? 1 : 0;
  p.ho = s.ho; p.wo = s.wo; p.taps = s.taps; p.oc = s.oc; p.cg = s.cg; p.ck = s.ck;
  p.tile_h = th; p.tile_w = tw; p.halo = halo; p.chunk = chunk;
  p.bhalo = bhalo < 0 ? halo : bhalo;
  // offset-conv chunk: at most four 16-byte k-steps per lane half (64 bf16
  // or 32 fp32 channels), the same in every plan of a layer so its offsets
  // are summed in one order
  const int amax = d.dtype == DEFT_BF16 ? 64 : 32;
  p.chunk_a = d.c_in % amax == 0 ? amax : (d.c_in % 32 == 0 ? 32 : 16);
  p.gw = 1;
  p.gsplit = d.offset_groups / p.gw;
  p.tiles_h = (s.ho + th - 1) / th;
  p.tiles_w = (s.wo + tw - 1) / tw;
  p.num_tiles = d.n * p.tiles_h * p.tiles_w;
  p.num_wg = p.num_tiles * p.gsplit;
  const int ocw = 2 * p.gw * s.taps;
  p.mblocks = (ocw + 31) / 32;
  p.oc_pad = (s.oc + 31) / 32 * 32 + 32;
  p.foot_h = (th - 1) * d.stride_h + (d.kh - 1) * d.dil_h + 1;
  p.foot_w = (tw - 1) * d.stride_w + (d.kw - 1) * d.dil_w + 1;
  p.reg_h = std::min(p.foot_h + 2 * halo + 1, d.h + 2);
  p.reg_w = std::min(p.foot_w + 2 * halo + 1, d.w + 2);
  const int vec = d.dtype == DEFT_BF16 ? 8 : 4;
  p.pstr = chunk + vec;
  p.pstr_a = p.chunk_a + vec;
  const int pt = th * tw;
  const int region = std::max({p.foot_h * p.foot_w * p.pstr_a * s.esz, p.reg_h * p.reg_w * p.pstr * s.esz,
                               4 * ocw * pt * 4});
  p.lds_region = 0;
  p.stage_d = 0;
  if (direct) {
    // offsets, then one region shared in turn by the double-buffered
    // footprint staging (256 * stage_d 16-byte slots per buffer), the
    // phase-A partial sums and the tap table (int4 corner offsets, float4
    // weights, int column offset)
    p.stage_d = (p.foot_h * p.foot_w * (p.chunk_a / vec) + 255) / 256;
    if (p.stage_d > 7) return false;
    p.lds_off = 0;
    p.lds_info = align16(ocw * pt * 4);
    p.lds_region = p.lds_info;
    p.lds_total = p.lds_info + std::max({4 * ocw * pt * 4, 36 * s.taps * pt, 2 * p.stage_d * 4096});
  } else {
    p.lds_off = align16(region);
    p.lds_info = p.lds_off + align16(ocw * pt * 4);
    p.lds_total = p.lds_info + align16(p.gw * s.taps * pt * 8) + p.gw * s.taps * pt * 16;  // tap table + weights
  }
  if (p.lds_total > p.max_lds) return false;
  p.num_btiles = 0; p.list_cap = 0; p.woff_bands = 1;
  if (!layout_backward(p)) p.chunk_b = 0;
  // workspace
  const size_t P = (size_t)d.n * s.ho * s.wo;
  p.kk_pad = (s.oc * s.taps + 15) / 16 * 16;
  size_t o = 0;
  p.ws_wt = o; o = align256(o + (size_t)d.c_out * s.ck * s.esz);
  p.ws_woff = o;
  o = align256(o + (size_t)std::max(p.oc_pad, 32 * d.offset_groups) * s.ck * s.esz);  // rows or fragments
  p.ws_cols = o; o = align256(o + P * s.ck * s.esz);
  p.ws_xh = o;
  if (direct) o = align256(o + (size_t)d.n * ((size_t)d.h * d.w + 1) * d.c_in * s.esz);
  p.igemm = 0;
  p.ws_offs = o;
  if (direct && deft::igemm_supported(p)) o = align256(o + P * s.oc * 4);  // offsets when the caller keeps none
  p.ws_fwd_end = o;
  p.ws_w2 = o; o = align256(o + (size_t)s.ck * d.c_out * s.esz);
  p.ws_wofft = o; o = align256(o + (size_t)d.c_in * p.kk_pad * s.esz);
  p.ws_dcol = o; o = align256(o + P * s.ck * s.esz);
  p.ws_dx32 = o; o = align256(o + (size_t)d.n * d.c_in * d.h * d.w * 4);
  p.ws_doff = o; o = align256(o + P * s.oc * 4);
  // bf16: dOffset rounded once more, as the offset-weight backward reads it
  p.ws_doff16 = o; if (d.dtype == DEFT_BF16) o = align256(o + P * s.oc * 2);
  p.ws_list = o;
  o = align256(o + (size_t)p.num_btiles * d.offset_groups * (p.list_cap + 64) * 16);
  p.ws_lcount = o; o = align256(o + (size_t)p.num_btiles * d.offset_groups * 4);
  // dOffset partials (one per backward channel chunk) followed by one word
  // for max |dCol|; both zeroed by the backward's prep kernel
  p.ws_doffp = o;
  const size_t nchunks = p.chunk_b ? (size_t)(s.cg / p.chunk_b) : 1;
  p.ws_maxbits = p.ws_doffp + nchunks * P * s.oc * 4;
  o = align256(p.ws_maxbits + 16);
  p.gemm_dl = deft::gemm_dl_supported(p) ? 1 : 0;
  if (p.gemm_dl) {
    deft::gemm_dl_dw_split(p, &p.dw_splits, &p.dw_kper);
  } else {
    p.dw_splits = d.n;
    p.dw_kper = s.ho * s.wo;
  }
  p.ws_dwpart = o; o = align256(o + (size_t)p.dw_splits * d.c_out * s.ck * 4);
  p.ws_dwoffpart = o; o = align256(o + (size_t)d.n * p.woff_bands * s.oc * s.ck * 4);
  // bias partials: [Cout][N] dY sums, then [Oc][N][blocks of 256 pixels] dOffset sums
  p.ws_biaspart = o; o = align256(o + ((size_t)d.c_out + (size_t)s.oc * (((size_t)s.ho * s.wo + 255) / 256)) * d.n * 4);
  p.ws_train_end = o;
  return true;
}

// Share of (not fully outside) taps whose corner lies beyond `halo` pixels.
// Without a histogram, or with one that counted no tap at all, default
// shares.
double miss_fraction(const uint32_t* hist, int len, int halo) {
  double in = 0, tot = 0, all = 0;
  for (int i = 0; hist && i < len; ++i) {
    all += hist[i];
    if (i < len - 1) tot += hist[i];
    if (i <= halo && i < len - 2) in += hist[i];
  }
  if (!hist || len < 3 || all <= 0) return halo >= 2 ? 0.01 : (halo == 1 ? 0.3 : 0.7);
  return tot > 0 ? 1.0 - in / tot : 0.0;
}

// Backward halo: every tap whose corner lies beyond it goes to the
// backward's slow path (one wave per tap, global atomics), measured at tens
// of nanoseconds per tap and a tail of several microseconds for even a few
// dozen taps, while each extra pixel of halo only widens the candidate scan
// of the sampling backward by about one percent.  So it is the smallest halo
// that leaves no more than 1e-5 of the taps outside, apart from those in the
// histogram's open-ended last distance bin, which no halo it describes can
// take in (capped at 16).  Without a histogram, or with one that counted no
// tap: 4 pixels.
int backward_halo(const uint32_t* hist, int len) {
  if (!hist || len < 3) return 4;
  double tot = 0;
  for (int i = 0; i < len - 1; ++i) tot += hist[i];
  if (tot + hist[len - 1] <= 0) return 4;  // a histogram that counted no tap says nothing
  const double allowed = hist[len - 2] + 1e-5 * tot;
  double in = 0;
  const int hmax = std::min(16, len - 3);
  for (int h = 0; h <= hmax; ++h) {
    in += hist[h];
    if (tot - in <= allowed) return h;
  }
  return hmax;
}

// Planner: pick (tile, halo, chunk) minimising a byte-cost estimate of the
// fused kernel: the columns it must write, the input staged into LDS (served
// mostly from L2, weighted down), the taps outside the halo, each of which
// reads its four corners per channel from global memory (weighted by 0.4 of
// those bytes: measured on 64 x 64 fp32 with offsets of about a pixel, a
// third of the taps outside the halo costs the kernel about 4 %, while on the
// 28 x 28 four-group layer with offsets of about 4 px, halo 1 against halo 8
// costs 60 %), and a fixed cost per channel-chunk pass, divided by the
// fraction of the machine the launch keeps busy.  A region so large that only one workgroup fits a CU
// leaves four waves to hide the gather latency: measured 1.7 to 1.8 times
// slower than two per CU, whatever the halo saves.
int plan_auto(deft_plan& best, const deft_desc& d, const uint32_t* hist, int hist_len, bool need_bwd = true) {
  const Shape s = shape_of(d);
  const DeviceLimits lim = device_limits();
  static const int tiles[][2] = {{8, 8}, {4, 16}, {16, 4}, {8, 4}, {4, 8}, {4, 4}, {2, 16}, {16, 2}, {2, 8}, {1, 16}};
  double best_cost = 1e300;
  bool found = false;
  const double samples = (double)d.n * s.ho * s.wo * s.taps * d.c_in;
  const double col_bytes = samples * s.esz;
  for (auto& t : tiles) {
    for (int halo = 0; halo <= 16; ++halo) {
      for (int chunk = 64; chunk >= 16; chunk /= 2) {
        if (s.cg % chunk) continue;
        deft_plan p = blank_plan(d, lim);
        if (!layout_plan(p, t[0], t[1], halo, chunk) || (need_bwd && p.chunk_b == 0)) continue;
        const double miss = miss_fraction(hist, hist_len, halo);
        const double pt = (double)t[0] * t[1];
        const double per_tile_stage = (double)p.reg_h * p.reg_w * s.cg + (double)p.foot_h * p.foot_w * d.c_in;
        const double stage_bytes = (double)p.num_wg * per_tile_stage * s.esz;
        const double miss_bytes = 0.4 * miss * samples * 4.0 * s.esz;
        const int occ = std::max(1, std::min(4, p.max_lds / std::max(p.lds_total, 1)));
        const double slots = (double)p.cus * occ;
        const double waves = std::ceil(p.num_wg / slots);
        const double busy = p.num_wg > 0 ? p.num_wg / (waves * slots) : 1.0;
        // each channel-chunk pass of a workgroup pays a staging round trip and
        // two barriers, about as much as moving 16 KB
        const double passes = (double)p.num_wg * p.gw * (s.cg / chunk) + (double)p.num_wg * (d.c_in / p.chunk_a);
        double cost = (col_bytes + 0.25 * stage_bytes + miss_bytes + passes * 16384.0) / std::max(busy, 0.05);
        if (occ == 1) cost *= 1.7;
        if (pt < 32) cost *= 1.1;  // phase-A MFMA blocks half empty
        if (cost < best_cost * 0.999) {
          best_cost = cost;
          best = p;
          found = true;
        }
      }
    }
  }
  if (!found) return need_bwd ? plan_auto(best, d, hist, hist_len, false) : DEFT_ERR_UNSUPPORTED;
  // Direct gather where supported: no LDS halo; the tile only sets the
  // forward's launch shape.  Every tile of 32..64 pixels is a candidate (fewer only when the
  // output is smaller).  Cost: the columns of every pixel slot the launch
  // covers, including the empty slots of ragged edge tiles (their offset conv
  // and tap work is done anyway); the footprint each workgroup stages for its
  // offset conv (served from the L2, weighted down); a fixed cost per
  // workgroup for its offset weights and staging round trips (about as much as
  // writing 64 KB of columns); all divided by the share of the machine the
  // launch keeps busy.  On 56 x 56 this prefers 7 x 7 (1024 workgroups, four
  // per CU) over 4 x 16, whose last tile column is half empty (measured 72.8
  // against 79.0 us).
  if (direct_ok(d)) {
    double dbest = 1e300;
    deft_plan bd;
    bool dfound = false;
    const double valid = (double)d.n * s.ho * s.wo * d.offset_groups;
    const int min_pt = std::min(32, s.ho * s.wo);
    for (int th = 1; th <= 16; ++th)
      for (int tw = 1; th * tw <= 64; ++tw) {
        if (th * tw < min_pt) continue;
        deft_plan p = blank_plan(d, lim);
        if (!layout_plan(p, th, tw, best.halo, s.cg, true) || (need_bwd && p.chunk_b == 0)) continue;
        const int occ = std::max(1, std::min(4, p.max_lds / std::max(p.lds_total, 1)));
        const double slots = (double)p.cus * occ;
        const double waves = std::ceil(p.num_wg / slots);
        const double busy = p.num_wg > 0 ? p.num_wg / (waves * slots) : 1.0;
        const double padded = (double)p.num_wg * th * tw;
        const double stage = (double)p.num_wg * p.foot_h * p.foot_w * d.c_in * s.esz;
        // fewer than four workgroups resident per CU hide less latency (fp32
        // on 64 x 64: 32-pixel tiles, four per CU, 58-61 us; 64-pixel tiles,
        // two per CU, 66-68 us)
        const double resident = std::min<double>(occ, std::ceil((double)p.num_wg / std::max(p.cus, 1)));
        const double lat = 1.0 + 0.25 * (4.0 / std::max(resident, 1.0) - 1.0);
        const double cost =
            lat * (col_bytes * padded / std::max(valid, 1.0) + 0.25 * stage + (double)p.num_wg * 65536.0) /
            std::max(busy, 0.05);
        if (cost < dbest * 0.999) {
          dbest = cost;
          bd = p;
          dfound = true;
        }
      }
    if (dfound) best = bd;
  }
  // the backward's halo is set by the tap distances alone
  const int bh = backward_halo(hist, hist_len);
  deft_plan q = blank_plan(d, lim);
  if (layout_plan(q, best.tile_h, best.tile_w, best.halo, best.chunk, best.direct != 0, bh) &&
      (q.chunk_b != 0 || !need_bwd))
    best = q;
  best.est_miss = miss_fraction(hist, hist_len, best.bhalo);
  return DEFT_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Timing {
  bool active = false;
  int used = 0;
  std::vector<hipEvent_t> ev;       // 2 per launch
  std::vector<const char*> names;
  std::vector<float> ms;
  // events are not destroyed at thread exit: that may run after the HIP
  // runtime has shut down; the process releases them
};
thread_local Timing g_timing;

}  // namespace

namespace deft {
int report_hip_error(hipError_t e) { return hip_fail(e); }

void timing_before(hipStream_t s, const char* name) {
  Timing& t = g_timing;
  if (!t.active || 2 * (size_t)t.used + 1 >= t.ev.size()) return;
  t.names[t.used] = name;
  (void)hipEventRecord(t.ev[2 * t.used], s);
}
void timing_after(hipStream_t s) {
  Timing& t = g_timing;
  if (!t.active || 2 * (size_t)t.used + 1 >= t.ev.size()) return;
  (void)hipEventRecord(t.ev[2 * t.used + 1], s);
  ++t.used;
}
}  // namespace deft

extern "C" {

int deft_desc_validate(const deft_desc* d) { return validate(d); }

int deft_plan_create(const deft_desc* d, const uint32_t* halo_hist, int hist_len, deft_plan** out) {
  if (!out) return DEFT_ERR_NULLPTR;
  const int v = validate(d);
  if (v) return v;
  deft_plan* p = new (std::nothrow) deft_plan();
  if (!p) return DEFT_ERR_UNSUPPORTED;
  const int r = plan_auto(*p, *d, halo_hist, halo_hist ? hist_len : 0);
  if (r) {
    delete p;
    return r;
  }
  *out = p;
  return DEFT_OK;
}

int deft_plan_create_forced(const deft_desc* d, int tile_h, int tile_w, int halo, int chunk, deft_plan** out) {
  if (!out) return DEFT_ERR_NULLPTR;
  const int v = validate(d);
  if (v) return v;
  const Shape s = shape_of(*d);
  if (tile_h < 1 || tile_w < 1 || tile_h * tile_w > 64 || halo < 0 || halo > 32) return DEFT_ERR_PLAN;
  if (chunk != 0 && chunk != -1 && chunk != -2 && (chunk < 16 || chunk > 64 || chunk % 16 || s.cg % chunk))
    return DEFT_ERR_PLAN;
  if ((chunk == -1 || chunk == -2) && !direct_ok(*d)) return DEFT_ERR_PLAN;
  deft_plan* p = new (std::nothrow) deft_plan();
  if (!p) return DEFT_ERR_UNSUPPORTED;
  *p = blank_plan(*d, device_limits());
  p->num_btiles = 0;
  bool ok = false;
  if (chunk == -1 || chunk == -2) {
    ok = layout_plan(*p, tile_h, tile_w, halo, s.cg, true);
    if (ok && chunk == -2) {
      ok = deft::igemm_supported(*p);
      p->igemm = ok ? 1 : 0;
    }
  } else if (chunk != 0) {
    ok = layout_plan(*p, tile_h, tile_w, halo, chunk);
  } else {
    for (int c = 64; c >= 16 && !ok; c /= 2)
      if (s.cg % c == 0) ok = layout_plan(*p, tile_h, tile_w, halo, c);
  }
  if (!ok) {
    delete p;
    return DEFT_ERR_PLAN;
  }
  p->est_miss = -1.0;
  *out = p;
  return DEFT_OK;
}

int deft_plan_get_info(const deft_plan* p, deft_plan_info* info) {
  if (!p || !info) return DEFT_ERR_NULLPTR;
  info->tile_h = p->tile_h; info->tile_w = p->tile_w; info->halo = p->halo; info->chunk = p->chunk;
  info->bwd_halo = p->bhalo;
  info->groups_per_wg = p->gw; info->num_workgroups = p->num_wg;
  info->ho = p->ho; info->wo = p->wo; info->oc = p->oc;
  info->lds_bytes = p->lds_total;
  info->est_miss_fraction = p->est_miss;
  info->ws_forward = p->ws_fwd_end;
  info->ws_training = p->ws_train_end;
  info->ws_cols_offset = p->ws_cols;
  info->bwd_tile_h = p->btile_h;
  info->bwd_tile_w = p->btile_w;
  info->bwd_chunk = p->chunk_b;
  info->gemm_direct = p->gemm_dl;
  info->gather_direct = p->direct;
  info->gather_gemm = p->igemm;
  info->dw_splits = p->dw_splits;
  return DEFT_OK;
}

void deft_plan_destroy(deft_plan* p) { delete p; }

size_t deft_workspace_bytes(const deft_plan* p, int training) {
  if (!p) return 0;
  return training ? p->ws_train_end : p->ws_fwd_end;
}

// The forward in the fused form (one sampling launch computes the offsets and
// the columns) or in the unfused three-operator form (offset conv -> offsets
// in HBM -> sampling -> GEMM), which needs the offsets buffer.
static int forward_impl(const deft_plan* p, const void* x, const void* w_off, const void* b_off, const void* w,
                        const void* b, void* y, float* offsets_out, void* workspace, size_t ws_bytes, void* stream,
                        bool fused, uint32_t* hist = nullptr, int hist_len = 0) {
  if (!p) return DEFT_ERR_NULLPTR;
  if (p->d.n == 0) return DEFT_OK;  // empty batch: nothing is read or written
  if (!x || !w_off || !w || !y) return DEFT_ERR_NULLPTR;
  if (!fused && !offsets_out) return DEFT_ERR_NULLPTR;
  if (!workspace || ws_bytes < p->ws_fwd_end) return DEFT_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w_off) || !aligned16(w) || !aligned16(y) || !aligned16(workspace) ||
      (offsets_out && !aligned16(offsets_out)))
    return DEFT_ERR_ALIGN;
  const size_t esz = p->d.dtype == DEFT_BF16 ? 2 : 4;
  if (((uintptr_t)b_off % esz) || ((uintptr_t)b % esz)) return DEFT_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hipError_t e = deft::launch_prep_forward(*p, w, w_off, ws + p->ws_wt, ws + p->ws_woff, x, ws + p->ws_xh, st);
  if (e != hipSuccess) return hip_fail(e);
  deft::SampleArgs a;
  a.x = x; a.woff_p = ws + p->ws_woff; a.b_off = b_off; a.off_out = offsets_out;
  a.cols = ws + p->ws_cols;
  a.xh = p->direct ? ws + p->ws_xh : nullptr;
  a.hist = hist;
  a.hist_len = hist_len;
  if (fused && p->igemm) {
    // offset conv, then the gather fused into the main GEMM (y and columns)
    float* off = offsets_out ? offsets_out : (float*)(ws + p->ws_offs);
    a.off_out = off;
    e = deft::launch_sample(*p, deft::kOffsetsMode, a, st);
    if (e != hipSuccess) return hip_fail(e);
    e = deft::launch_igemm(*p, ws + p->ws_xh, off, ws + p->ws_wt, b, y, ws + p->ws_cols, st);
    if (e != hipSuccess) return hip_fail(e);
    return DEFT_OK;
  }
  if (fused) {
    e = deft::launch_sample(*p, deft::kFusedMode, a, st);
  } else {
    e = deft::launch_sample(*p, deft::kOffsetsMode, a, st);
    if (e != hipSuccess) return hip_fail(e);
    a.off_out = nullptr;
    a.off_in = offsets_out;
    e = deft::launch_sample(*p, deft::kSampleMode, a, st);
  }
  if (e != hipSuccess) return hip_fail(e);
  e = deft::launch_gemm_forward(*p, ws + p->ws_wt, ws + p->ws_cols, b, y, st);
  if (e != hipSuccess) return hip_fail(e);
  return DEFT_OK;
}

int deft_forward(const deft_plan* p, const void* x, const void* w_off, const void* b_off, const void* w,
                 const void* b, void* y, float* offsets_out, void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(p, x, w_off, b_off, w, b, y, offsets_out, workspace, ws_bytes, stream, true);
}

int deft_forward_hist(const deft_plan* p, const void* x, const void* w_off, const void* b_off, const void* w,
                      const void* b, void* y, float* offsets_out, void* workspace, size_t ws_bytes, uint32_t* hist,
                      int hist_len, void* stream) {
  if (!p) return DEFT_ERR_NULLPTR;
  if (hist_len < 3 || hist_len > 64) return DEFT_ERR_BAD_DESC;
  if (!hist && p->d.n > 0) return DEFT_ERR_NULLPTR;
  if ((uintptr_t)hist & 3u) return DEFT_ERR_ALIGN;
  return forward_impl(p, x, w_off, b_off, w, b, y, offsets_out, workspace, ws_bytes, stream, true, hist, hist_len);
}

int deft_forward_unfused(const deft_plan* p, const void* x, const void* w_off, const void* b_off, const void* w,
                         const void* b, void* y, float* offsets, void* workspace, size_t ws_bytes, void* stream) {
  return forward_impl(p, x, w_off, b_off, w, b, y, offsets, workspace, ws_bytes, stream, false);
}

int deft_backward(const deft_plan* p, const void* x, const void* w_off, const void* w, const float* offsets,
                  const void* dy, void* workspace, size_t ws_bytes, void* dx, void* dw_off, void* db_off, void* dw,
                  void* db, void* stream) {
  if (!p) return DEFT_ERR_NULLPTR;
  if (p->d.n == 0) return DEFT_OK;  // empty batch
  if (!x || !w_off || !w || !offsets || !dy || !dx || !dw_off || !dw) return DEFT_ERR_NULLPTR;
  if (!workspace || ws_bytes < p->ws_train_end) return DEFT_ERR_WORKSPACE;
  if (p->chunk_b == 0) return DEFT_ERR_PLAN;
  if (!aligned16(x) || !aligned16(w_off) || !aligned16(w) || !aligned16(offsets) || !aligned16(dy) ||
      !aligned16(dx) || !aligned16(dw_off) || !aligned16(dw) || !aligned16(workspace))
    return DEFT_ERR_ALIGN;
  const size_t esz = p->d.dtype == DEFT_BF16 ? 2 : 4;
  if (((uintptr_t)db_off % esz) || ((uintptr_t)db % esz)) return DEFT_ERR_ALIGN;
  if (p->d.n == 0) return DEFT_OK;
  deft::BackwardArgs a;
  a.x = x; a.w_off = w_off; a.w = w; a.offsets = offsets; a.dy = dy; a.dx = dx; a.dw_off = dw_off;
  a.db_off = db_off; a.dw = dw; a.db = db; a.ws = (char*)workspace;
  const hipError_t e = deft::launch_backward(*p, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return DEFT_OK;
}

int deft_debug_sample_index(const deft_desc* d, const float* offsets, int32_t* y0, int32_t* x0, uint8_t* mask,
                            void* stream) {
  const int v = validate(d);
  if (v) return v;
  if (!offsets || !y0 || !x0 || !mask) return DEFT_ERR_NULLPTR;
  if (((uintptr_t)offsets & 3u) || ((uintptr_t)y0 & 3u) || ((uintptr_t)x0 & 3u)) return DEFT_ERR_ALIGN;
  const Shape s = shape_of(*d);
  const hipError_t e = deft::launch_sample_index(*d, s.ho, s.wo, offsets, y0, x0, mask, (hipStream_t)stream);
  return e == hipSuccess ? DEFT_OK : hip_fail(e);
}

int deft_debug_sample(const deft_plan* p, const void* x, const float* offsets, void* cols, void* stream) {
  if (!p) return DEFT_ERR_NULLPTR;
  if (p->d.n == 0) return DEFT_OK;
  if (!x || !offsets || !cols) return DEFT_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(cols) || ((uintptr_t)offsets & 3u)) return DEFT_ERR_ALIGN;
  if (p->d.n == 0) return DEFT_OK;
  deft::SampleArgs a;
  a.x = x; a.woff_p = nullptr; a.b_off = nullptr; a.off_in = offsets; a.off_out = nullptr; a.cols = cols;
  if (p->direct) {
    // sampling from given offsets always uses the LDS tile + halo kernel
    // (it has no workspace for the channel-minor copy)
    deft_plan q = blank_plan(p->d, DeviceLimits{});
    q.cus = p->cus;
    q.max_lds = p->max_lds;
    bool ok = false;
    for (int c = 64; c >= 16 && !ok; c /= 2)
      if (p->cg % c == 0) ok = layout_plan(q, p->tile_h, p->tile_w, p->halo, c);
    if (!ok) return DEFT_ERR_PLAN;
    const hipError_t e = deft::launch_sample(q, deft::kSampleMode, a, (hipStream_t)stream);
    return e == hipSuccess ? DEFT_OK : hip_fail(e);
  }
  const hipError_t e = deft::launch_sample(*p, deft::kSampleMode, a, (hipStream_t)stream);
  return e == hipSuccess ? DEFT_OK : hip_fail(e);
}

int deft_halo_histogram(const deft_desc* d, const float* offsets, uint32_t* hist, int hist_len, void* stream) {
  const int v = validate(d);
  if (v) return v;
  if (!offsets || !hist) return DEFT_ERR_NULLPTR;
  if (hist_len < 3 || hist_len > 64) return DEFT_ERR_BAD_DESC;
  if (((uintptr_t)offsets & 3u) || ((uintptr_t)hist & 3u)) return DEFT_ERR_ALIGN;
  const Shape s = shape_of(*d);
  const hipError_t e = deft::launch_halo_hist(*d, s.ho, s.wo, offsets, hist, hist_len, (hipStream_t)stream);
  return e == hipSuccess ? DEFT_OK : hip_fail(e);
}

int deft_dwconv1d_forward(const float* x, const float* w, float* y, int batch, int steps, int channels, int ksize,
                          int dilation, void* stream) {
  if (batch < 0 || steps < 0 || channels < 4 || channels % 4 || ksize < 1 || ksize > 256 || dilation < 1)
    return DEFT_ERR_BAD_DESC;
  const long long len = (long long)steps + (long long)dilation * (ksize - 1);
  if (len > 0x7fffffffLL) return DEFT_ERR_BAD_DESC;
  if (batch == 0 || steps == 0) return DEFT_OK;
  if (!x || !w || !y) return DEFT_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return DEFT_ERR_ALIGN;
  const hipError_t e =
      deft::launch_dwconv1d(x, w, y, batch, steps, channels, ksize, dilation, (hipStream_t)stream);
  return e == hipSuccess ? DEFT_OK : hip_fail(e);
}

int deft_dwpw1d_forward(const float* x, const float* w_dw, const float* w_pw, float* z, int batch, int steps,
                        int channels, int out_channels, int ksize, int dilation, void* stream) {
  if (batch < 0 || steps < 0 || channels < 32 || channels % 32 || out_channels < 32 || out_channels % 32 ||
      ksize < 1 || ksize > 256 || dilation < 1)
    return DEFT_ERR_BAD_DESC;
  const long long len = (long long)steps + (long long)dilation * (ksize - 1);
  if (len > 0x7fffffffLL) return DEFT_ERR_BAD_DESC;
  if (batch == 0 || steps == 0) return DEFT_OK;
  if (!x || !w_dw || !w_pw || !z) return DEFT_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(w_dw) || !aligned16(w_pw) || !aligned16(z)) return DEFT_ERR_ALIGN;
  const hipError_t e = deft::launch_dwpw1d(x, w_dw, w_pw, z, batch, steps, channels, out_channels, ksize, dilation,
                                           (hipStream_t)stream);
  return e == hipSuccess ? DEFT_OK : hip_fail(e);
}

int deft_timing_start(int capacity) {
  if (capacity < 1) return DEFT_ERR_BAD_DESC;
  Timing& t = g_timing;
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto& e : t.ev) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      t.ev.clear();
      t.active = false;
      return hip_fail(r);
    }
  }
  t.names.assign(capacity, "");
  t.ms.clear();
  t.used = 0;
  t.active = true;
  return DEFT_OK;
}

int deft_timing_stop(void) {
  Timing& t = g_timing;
  t.active = false;
  t.ms.assign(t.used, 0.f);
  if (t.used == 0) return DEFT_OK;
  hipError_t r = hipEventSynchronize(t.ev[2 * t.used - 1]);
  if (r != hipSuccess) return hip_fail(r);
  for (int i = 0; i < t.used; ++i) {
    r = hipEventElapsedTime(&t.ms[i], t.ev[2 * i], t.ev[2 * i + 1]);
    if (r != hipSuccess) return hip_fail(r);
  }
  return DEFT_OK;
}

int deft_timing_count(void) { return (int)g_timing.ms.size(); }

int deft_timing_get(int i, const char** name, float* ms) {
  const Timing& t = g_timing;
  if (i < 0 || i >= (int)t.ms.size()) return DEFT_ERR_BAD_DESC;
  if (name) *name = t.names[i];
  if (ms) *ms = t.ms[i];
  return DEFT_OK;
}

const char* deft_error_string(int code) {
  switch (code) {
    case DEFT_OK: return "ok";
    case DEFT_ERR_BAD_DESC: return "invalid descriptor (sizes, kernel, stride, dilation or padding)";
    case DEFT_ERR_GROUPS: return "offset_groups must be >= 1 and divide c_in";
    case DEFT_ERR_SHAPE: return "output height or width is < 1";
    case DEFT_ERR_NULLPTR: return "a required pointer is NULL";
    case DEFT_ERR_WORKSPACE: return "workspace missing or smaller than deft_workspace_bytes";
    case DEFT_ERR_DTYPE: return "dtype must be DEFT_F32 or DEFT_BF16";
    case DEFT_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case DEFT_ERR_HIP: return "HIP runtime error (see deft_last_hip_error)";
    case DEFT_ERR_PLAN: return "forced tile/halo/chunk outside the supported range";
    case DEFT_ERR_UNSUPPORTED: return "unsupported shape (channels per offset group must be a multiple of 16)";
    case DEFT_ERR_SCRATCH:
      return "the forward needs more scratch than the no-allocation entry point's static buffer holds "
             "(DEFT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error";
  }
}

const char* deft_last_hip_error(void) { return g_last_hip; }

}  // extern "C"
