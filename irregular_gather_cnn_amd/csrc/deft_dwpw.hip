// Fused depthwise + pointwise 1-D convolution (fp32, channel-minor layout)
// for gfx950: z[b][t][o] = sum_c w_pw[c][o] * (sum_k w_dw[k][c] * x[b][t + k*d][c]).
//
// The FCM abstract fuses a depthwise convolution with the pointwise (1x1)
// convolution that follows it so that the depthwise output never goes to
// memory.  Here the depthwise result is produced where the pointwise GEMM
// consumes it: a workgroup owns 64 time steps x 512 output channels; for each
// slice of 32 input channels its threads compute the 64 x 32 depthwise
// outputs (K taps at dilation d, read through the caches) straight into LDS,
// stage the 32 x 512 slice of the pointwise weights next to them, and the
// 2 x 2 waves run the channel mix on the fp32 MFMA units (32x32x2, each wave
// 32 steps x 256 output channels).  The depthwise arithmetic is the fused
// multiply-add chain over k of the depthwise kernel; the mix sums in the
// MFMA's order.
#include "deft_device.h"
#include "deft_internal.h"

namespace deft {

namespace {
constexpr int kRT = 64, kOT = 512, kCS = 32;  // steps, output channels, input channels per stage
constexpr int kAS = kCS + 1;                  // LDS row stride of the depthwise tile (floats)
constexpr int kBS = kOT + 4;                  // LDS row stride of the weight slice (floats)
}  // namespace

struct DwpwParams {
  const float* x;     // [B][L][C]
  const float* wdw;   // [K][C]
  const float* wpw;   // [C][O]
  float* z;           // [B][T][O]
  int B, T, L, C, O, K, d, ttiles, otiles;
};

__global__ __launch_bounds__(256) void k_dwpw1d(const DwpwParams p) {
  extern __shared__ __align__(16) float smem_f[];
  float* Bs = smem_f;                 // [kCS][kBS]
  float* As = smem_f + kCS * kBS;     // [kRT][kAS]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int id = blockIdx.x;
  const int ot = id % p.otiles; id /= p.otiles;
  const int tt = id % p.ttiles;
  const int b = id / p.ttiles;
  const int t0 = tt * kRT, o0 = ot * kOT;
  const float* __restrict__ xb = p.x + (size_t)b * p.L * p.C;

  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  const int drow = tid >> 2, dcg = (tid & 3) * 8;  // depthwise: one step, 8 channels per thread
  const int dt = t0 + drow;
  for (int c0 = 0; c0 < p.C; c0 += kCS) {
    // depthwise outputs of this slice
    {
      float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
      if (dt < p.T) {
        const int c = c0 + dcg;
        for (int k = 0; k < p.K; ++k) {
          const float* xr = xb + ((size_t)dt + (size_t)k * p.d) * p.C + c;
          const float4 x0 = *(const float4*)xr, x1 = *(const float4*)(xr + 4);
          const float4 w0 = *(const float4*)(p.wdw + (size_t)k * p.C + c);
          const float4 w1 = *(const float4*)(p.wdw + (size_t)k * p.C + c + 4);
          a0.x = __builtin_fmaf(w0.x, x0.x, a0.x); a0.y = __builtin_fmaf(w0.y, x0.y, a0.y);
          a0.z = __builtin_fmaf(w0.z, x0.z, a0.z); a0.w = __builtin_fmaf(w0.w, x0.w, a0.w);
          a1.x = __builtin_fmaf(w1.x, x1.x, a1.x); a1.y = __builtin_fmaf(w1.y, x1.y, a1.y);
          a1.z = __builtin_fmaf(w1.z, x1.z, a1.z); a1.w = __builtin_fmaf(w1.w, x1.w, a1.w);
        }
      }
      float* ar = As + drow * kAS + dcg;
      ar[0] = a0.x; ar[1] = a0.y; ar[2] = a0.z; ar[3] = a0.w;
      ar[4] = a1.x; ar[5] = a1.y; ar[6] = a1.z; ar[7] = a1.w;
    }
    // pointwise weights of this slice: 32 rows x 512 columns, float4 per thread x 16
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = tid + 256 * j;  // float4 index in the 32 x 128 grid
      const int r = e >> 7, c4 = e & 127;
      const int o = o0 + c4 * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (o < p.O) v = *(const float4*)(p.wpw + (size_t)(c0 + r) * p.O + o);
      *(float4*)(Bs + r * kBS + c4 * 4) = v;
    }
    __syncthreads();
    // channel mix: A [step][channel] x B [channel][output]
#pragma unroll 4
    for (int kk = 0; kk < kCS / 2; ++kk) {
      const int kr = 2 * kk + (lane >> 5);
      const float a = As[(wm * 32 + (lane & 31)) * kAS + kr];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float bv = Bs[kr * kBS + wn * 256 + j * 32 + (lane & 31)];
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv, acc[j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // element r of block j: step t0 + wm*32 + acc_row(lane, r), output o0 + wn*256 + j*32 + lane%32
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int o = o0 + wn * 256 + j * 32 + (lane & 31);
    if (o >= p.O) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + wm * 32 + acc_row(lane, r);
      if (t < p.T) p.z[((size_t)b * p.T + t) * p.O + o] = acc[j][r];
    }
  }
}

hipError_t launch_dwpw1d(const float* x, const float* wdw, const float* wpw, float* z, int B, int T, int C, int O,
                         int K, int d, hipStream_t st) {
  DwpwParams p;
  p.x = x; p.wdw = wdw; p.wpw = wpw; p.z = z;
  p.B = B; p.T = T; p.C = C; p.O = O; p.K = K; p.d = d;
  p.L = T + d * (K - 1);
  p.ttiles = (T + kRT - 1) / kRT;
  p.otiles = (O + kOT - 1) / kOT;
  const size_t grid = (size_t)B * p.ttiles * p.otiles;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  const int lds = (kCS * kBS + kRT * kAS) * 4;
  hipError_t e = hipFuncSetAttribute((const void*)k_dwpw1d, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  DEFT_LAUNCH("dwpw1d", k_dwpw1d, dim3((unsigned)grid), dim3(256), lds, st, p);
  return hipGetLastError();
}

}  // namespace deft
