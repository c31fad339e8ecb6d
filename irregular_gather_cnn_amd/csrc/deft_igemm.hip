// Whole-layer fusion of the deformable convolution's forward (bf16, gfx950):
// the bilinear gather feeds the main convolution's MFMA GEMM directly, so the
// GEMM never reads the deformed columns back from HBM.
//
// The DefT explainer page keeps the main convolution a library GEMM that
// reads the interpolated columns from memory ("This paper's idea", "Why it
// works": the column step stays a GEMM, which is efficient on its own).  Here
// the GEMM is hand-written, so its A operand can be produced where it is
// consumed: for every 32-deep slice of the column depth (one tap, 32
// channels), each workgroup gathers the four corners of its 128 pixels from
// the channel-minor copy of x (L2 / Infinity Cache resident), blends them
// with the bilinear weights of offsets already in HBM (written by the
// offset-conv launch, 3.6 MB), and writes the bf16 slice into LDS, where the
// 32x32x16 MFMAs take it together with a 256-row slice of the weights.  The
// columns are still stored (non-temporal), because the backward's weight
// gradient needs them, but nothing reads them again in the forward.
//
// Arithmetic is that of the sampling kernels: the same tap index, weights,
// blend order and bf16 rounding, so the columns are bit-identical to theirs;
// y differs from the two-kernel path only in the summation order of the GEMM.
//
// Layout per workgroup (256 threads = 2 x 2 waves): 128 pixels (rows m of the
// flattened N*Ho*Wo index) x 256 output channels (columns n); each wave owns
// 64 x 128 (2 x 4 blocks of 32 x 32).  Global loads go to registers one stage
// ahead (corners of stage s+1 and weights of stage s+1 are in flight while
// the MFMAs of stage s run), then to LDS; all loads are ordinary vector loads
// whose completion the compiler tracks.
#include "deft_device.h"
#include "deft_internal.h"

namespace deft {

namespace {

constexpr int kBM = 128, kBN = 256, kBK = 32;
constexpr int kARow = kBK * 2;           // bytes per LDS row (64)
constexpr int kABytes = kBM * kARow;     // 8 KB
constexpr int kBBytes = kBN * kARow;     // 16 KB
constexpr int kEpiStride = 64 * 2 + 16;  // bytes per transposed epilogue row (64 pixels + pad)
constexpr int kEpiBytes = 4 * 128 * kEpiStride;

struct IgemmParams {
  const bf16_t* xh;    // channel-minor x [N][H*W+1][Cin], pixel H*W zero
  const float* off;    // offsets [N][Oc][Ho][Wo]
  const bf16_t* wt;    // main weight [Cout][taps][Cin]
  const bf16_t* bias;  // nullable
  bf16_t* y;           // [N][Cout][Ho][Wo]
  bf16_t* cols;        // [N*Ho*Wo][taps][Cin]
  int Cin, H, W, Ho, Wo, KW, SH, SW, PH, PW, DH, DW, Cg, K2, Oc, Ck, Cout, M, HoWo, HW;
  int tilesM, tilesN, cpt, lds_off;
  FastDiv div_howo, div_wo, div_cpt;
};

__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// One pixel's gather state for the current (tap, group): element offsets of
// its four corners in the channel-minor image (out-of-image corners point at
// the zero pixel) and the bilinear weights.
struct Corner {
  int a[4];
  float w[4];
};

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_igemm(const IgemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* lA = smem;                     // [kBM][64 B]
  unsigned char* lB = smem + kABytes;           // [kBN][64 B]
  float* offl = (float*)(smem + p.lds_off);     // [Oc][kBM]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lb = xcd_swizzle(blockIdx.x, p.tilesM * p.tilesN);
  const int mt = lb / p.tilesN, nt = lb - mt * p.tilesN;
  const int m0 = mt * kBM, n0 = nt * kBN;

  // offsets of the tile's pixels
  for (int e = tid; e < p.Oc * kBM; e += 256) {
    const int o = e / kBM, r = e - o * kBM;
    const int q = m0 + r;
    float v = 0.f;
    if (q < p.M) {
      const int n = fdiv(q, p.div_howo), pp = q - n * p.HoWo;
      v = p.off[((size_t)n * p.Oc + o) * p.HoWo + pp];
    }
    offl[e] = v;
  }

  // this thread's two pixels (rows) and 8-channel chunk of every A slice
  const int cc = tid & 3;
  int row_q[2], row_by[2], row_bx[2], row_img[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (tid >> 2) + 64 * j;
    const int q = m0 + r;
    row_q[j] = q;
    if (q < p.M) {
      const int n = fdiv(q, p.div_howo), pp = q - n * p.HoWo;
      const int oh = fdiv(pp, p.div_wo), ow = pp - oh * p.Wo;
      row_img[j] = n * (p.HW + 1) * p.Cin;
      row_by[j] = oh * p.SH - p.PH;
      row_bx[j] = ow * p.SW - p.PW;
    } else {
      row_img[j] = 0; row_by[j] = 0; row_bx[j] = 0;
    }
  }
  const int zero_px = p.HW * p.Cin;
  __syncthreads();  // offl

  // corners of stage s for row j: tap t = s / cpt, channels ch .. ch+7
  auto corner = [&](int j, int t, int ch) {
    Corner c;
    const int r = (tid >> 2) + 64 * j;
    const int g = ch / p.Cg;
    const int ti = t / p.KW, tj = t - ti * p.KW;
    const int by = row_by[j] + ti * p.DH, bx = row_bx[j] + tj * p.DW;
    const float dy = offl[(2 * (g * p.K2 + t)) * kBM + r];
    const float dx = offl[(2 * (g * p.K2 + t) + 1) * kBM + r];
    const TapIndex ix = tap_index(by, bx, dy, dx, p.H, p.W);
    const int m = row_q[j] < p.M ? (int)corner_mask(ix, p.H, p.W) : 0;
    tap_weights(ix, c.w);
    const int b = ix.outside ? 0 : (ix.y0 * p.W + ix.x0) * p.Cin;
    const int base = row_img[j] + ch;
    c.a[0] = base + ((m & 1) ? b : zero_px);
    c.a[1] = base + ((m & 2) ? b + p.Cin : zero_px);
    c.a[2] = base + ((m & 4) ? b + p.W * p.Cin : zero_px);
    c.a[3] = base + ((m & 8) ? b + p.W * p.Cin + p.Cin : zero_px);
    return c;
  };

  uint4 ga[2][4];    // corner chunks of the next A slice
  float gw[2][4];    // their weights
  uint4 gb[4];       // next B slice (weights), rows (tid >> 2) + 64 j
  auto load_stage = [&](int s) {
    const int t = fdiv(s, p.div_cpt), c0 = (s - t * p.cpt) * kBK;
    const int ch = c0 + 8 * cc;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const Corner c = corner(j, t, ch);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ga[j][k] = *(const uint4*)(p.xh + c.a[k]);
        gw[j][k] = c.w[k];
      }
    }
    const int k0 = s * kBK + 8 * cc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + (tid >> 2) + 64 * j;
      gb[j] = n < p.Cout ? *(const uint4*)(p.wt + (size_t)n * p.Ck + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int s) {
    const int t = fdiv(s, p.div_cpt), c0 = (s - t * p.cpt) * kBK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = (tid >> 2) + 64 * j;
      float f00[8], f01[8], f10[8], f11[8], o8[8];
      unpack8(ga[j][0], f00);
      unpack8(ga[j][1], f01);
      unpack8(ga[j][2], f10);
      unpack8(ga[j][3], f11);
#pragma unroll
      for (int c = 0; c < 8; ++c) o8[c] = blend4(gw[j], f00[c], f01[c], f10[c], f11[c]);
      const uint4 v = make_uint4(pack_bf16x2(o8[0], o8[1]), pack_bf16x2(o8[2], o8[3]), pack_bf16x2(o8[4], o8[5]),
                                 pack_bf16x2(o8[6], o8[7]));
      *(uint4*)(lA + r * kARow + ((cc ^ swz(r)) << 4)) = v;
      if (row_q[j] < p.M) store16_nt(p.cols + (size_t)row_q[j] * p.Ck + t * p.Cin + c0 + 8 * cc, v);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (tid >> 2) + 64 * j;
      *(uint4*)(lB + r * kARow + ((cc ^ swz(r)) << 4)) = gb[j];
    }
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = p.Ck / kBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    if (s + 1 < nk) load_stage(s + 1);  // in flight during this stage's MFMAs
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 fa[2], fb[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31), c = 2 * ks + (lane >> 5);
        fa[i] = *(const uint4*)(lA + r * kARow + ((c ^ swz(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 128 + j * 32 + (lane & 31), c = 2 * ks + (lane >> 5);
        fb[j] = *(const uint4*)(lB + r * kARow + ((c ^ swz(r)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                              __builtin_bit_cast(bf16x8_t, fb[j]), acc[i][j], 0, 0,
                                                              0);
    }
    __syncthreads();  // every wave is done reading this stage
    if (s + 1 < nk) store_stage(s + 1);
    __syncthreads();
  }

  // epilogue: each wave transposes its 64 x 128 block through LDS so a lane
  // writes 8 consecutive pixels of one output channel (16 bytes of NCHW y)
  unsigned char* reg = smem + wave * 128 * kEpiStride;
  const int mw = m0 + wm * 64, nw = n0 + wn * 128;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nl = j * 32 + (lane & 31);
      const float add = (p.bias && nw + nl < p.Cout) ? bf16_to_f32(p.bias[nw + nl]) : 0.f;
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
  // 8 chunks of 16 bytes per channel row, 8 rows per pass
#pragma unroll 4
  for (int it = 0; it < 128 / 8; ++it) {
    const int nl = it * 8 + (lane >> 3), c = lane & 7;
    const int n = nw + nl, m = mw + c * 8;
    if (n >= p.Cout || m >= p.M) continue;
    const uint4 v = *(const uint4*)(reg + nl * kEpiStride + c * 16);
    const int img = fdiv(m, p.div_howo), pp = m - img * p.HoWo;
    store16_nt(p.y + ((size_t)img * p.Cout + n) * p.HoWo + pp, v);
  }
}

// The fused forward applies when the gather slices line up with the MFMA
// depth: bf16, direct gather (channel-minor copy), 32-channel slices inside
// one group, whole 8-pixel runs per image for the epilogue, 32-bit offsets.
bool igemm_supported(const deft_plan& p) {
  const deft_desc& d = p.d;
  if (d.dtype != DEFT_BF16 || !p.direct) return false;
  const size_t howo = (size_t)p.ho * p.wo, P = (size_t)d.n * howo;
  if (d.c_in % kBK || p.cg % kBK || howo % 8 || d.c_out % 8) return false;
  const size_t lim = 0x7ffffff0u;
  return (size_t)d.n * ((size_t)d.h * d.w + 1) * d.c_in < lim && P * p.ck < lim && (size_t)d.c_out * p.ck < lim &&
         (size_t)p.oc * kBM * 4 + kABytes + kBBytes <= 65536;
}

size_t igemm_lds_bytes(const deft_plan& p) {
  const size_t main = kABytes + kBBytes + (size_t)p.oc * kBM * 4;
  return main > (size_t)kEpiBytes ? main : (size_t)kEpiBytes;
}

hipError_t launch_igemm(const deft_plan& p, const void* xh, const float* off, const void* wt, const void* b,
                        void* y, void* cols, hipStream_t st) {
  IgemmParams q;
  const deft_desc& d = p.d;
  q.xh = (const bf16_t*)xh; q.off = off; q.wt = (const bf16_t*)wt; q.bias = (const bf16_t*)b;
  q.y = (bf16_t*)y; q.cols = (bf16_t*)cols;
  q.Cin = d.c_in; q.H = d.h; q.W = d.w; q.Ho = p.ho; q.Wo = p.wo; q.KW = d.kw; q.SH = d.stride_h; q.SW = d.stride_w;
  q.PH = d.pad_h; q.PW = d.pad_w; q.DH = d.dil_h; q.DW = d.dil_w; q.Cg = p.cg; q.K2 = p.taps; q.Oc = p.oc;
  q.Ck = p.ck; q.Cout = d.c_out; q.HoWo = p.ho * p.wo; q.M = d.n * q.HoWo; q.HW = d.h * d.w;
  q.tilesM = (q.M + kBM - 1) / kBM; q.tilesN = (d.c_out + kBN - 1) / kBN;
  q.cpt = d.c_in / kBK;
  q.lds_off = kABytes + kBBytes;
  q.div_howo = make_fastdiv(q.HoWo); q.div_wo = make_fastdiv(p.wo); q.div_cpt = make_fastdiv(q.cpt);
  const int lds = (int)igemm_lds_bytes(p);
  hipError_t e = hipFuncSetAttribute((const void*)k_igemm, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = q.tilesM * q.tilesN;
  if (grid == 0) return hipSuccess;
  DEFT_LAUNCH("fused_gather_gemm", k_igemm, dim3(grid), dim3(256), lds, st, q);
  return hipGetLastError();
}

}  // namespace deft
