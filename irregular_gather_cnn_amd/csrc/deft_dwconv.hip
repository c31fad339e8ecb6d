// Dilated depthwise 1-D convolution (fp32, channel-minor "NTC" layout) for
// gfx950: y[b][t][c] = sum_k w[k][c] * x[b][t + k*d][c], VALID padding.
//
// This is the workload of the JAX issue page on grouped and dilated
// convolutions: there, the depthwise form gets slower as the dilation grows,
// although it does less arithmetic.  Tiling along time breaks down under
// dilation because a tile of T_t outputs reads a window of T_t + d(K-1) input
// rows, mostly halo.  Here the time axis is split into its d phases instead:
// outputs whose step has residue r modulo d read only inputs with residue r,
// so each phase is an undilated K-tap convolution over a stride-d
// subsequence.  A workgroup owns P consecutive phases x TJ phase steps of one
// 64-channel slice and stages the (TJ + K - 1) x P input rows they need in LDS
// (for a fixed phase step the P phases are consecutive rows in memory, so the
// staging reads whole 256-byte runs), together with the K tap weights.  When
// a phase fits in one tile, every input row is staged once, whatever d is.
#include "deft_device.h"
#include "deft_internal.h"

namespace deft {

struct DwParams {
  const float4* x;  // [B][L][C/4]
  const float4* w;  // [K][C/4]
  float4* y;        // [B][T][C/4]
  int B, T, L, C4, K, d;
  int R, P, TJ, CV;          // non-empty phases, phases / steps / float4 lanes per tile
  int four;                  // 1: four phase steps per thread (enough work items for the workgroup)
  int pgroups, jtiles, cchunks;
};

__global__ __launch_bounds__(256) void k_dwconv1d(const DwParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int rows = p.TJ + p.K - 1;
  float4* xs = (float4*)smem;             // [rows][P][CV]
  float4* ws = xs + rows * p.P * p.CV;    // [K][CV]
  int id = blockIdx.x;
  const int cch = id % p.cchunks; id /= p.cchunks;
  const int jt = id % p.jtiles; id /= p.jtiles;
  const int pg = id % p.pgroups;
  const int b = id / p.pgroups;
  const int r0 = pg * p.P, j0 = jt * p.TJ, c40 = cch * p.CV;
  // phase r has (T - r + d - 1) / d outputs; the first phase of the tile has the most
  if (r0 >= p.R || j0 * p.d + r0 >= p.T) return;  // uniform: nothing to compute
  const size_t xb = (size_t)b * p.L * p.C4, yb = (size_t)b * p.T * p.C4;

  for (int e = threadIdx.x; e < p.K * p.CV; e += 256) {
    const int k = e / p.CV, v = e - k * p.CV;
    ws[e] = c40 + v < p.C4 ? p.w[(size_t)k * p.C4 + c40 + v] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int per_row = p.P * p.CV;
  for (int e = threadIdx.x; e < rows * per_row; e += 256) {
    const int il = e / per_row, rem = e - il * per_row;
    const int pl = rem / p.CV, v = rem - pl * p.CV;
    const int r = r0 + pl, i = j0 + il;
    const int n_r = r < p.R ? (p.T - r + p.d - 1) / p.d : 0;
    float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
    // rows past the phase's last window are never read by a valid output
    if (i < n_r + p.K - 1 && c40 + v < p.C4) val = p.x[xb + ((size_t)r + (size_t)p.d * i) * p.C4 + c40 + v];
    xs[e] = val;
  }
  __syncthreads();

  if (!p.four) {
    // short phases (large dilation and kernel): one output row per thread
    for (int e = threadIdx.x; e < p.TJ * per_row; e += 256) {
      const int jl = e / per_row, rem = e - jl * per_row;
      const int pl = rem / p.CV, v = rem - pl * p.CV;
      const int r = r0 + pl, j = j0 + jl;
      if (r >= p.R || c40 + v >= p.C4) continue;
      if (j >= (p.T - r + p.d - 1) / p.d) continue;
      const float4* xr = xs + (size_t)jl * per_row + pl * p.CV + v;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int k = 0; k < p.K; ++k) {
        const float4 xv = xr[(size_t)k * per_row], wv = ws[k * p.CV + v];
        acc.x = __builtin_fmaf(wv.x, xv.x, acc.x);
        acc.y = __builtin_fmaf(wv.y, xv.y, acc.y);
        acc.z = __builtin_fmaf(wv.z, xv.z, acc.z);
        acc.w = __builtin_fmaf(wv.w, xv.w, acc.w);
      }
      p.y[yb + ((size_t)r + (size_t)p.d * j) * p.C4 + c40 + v] = acc;
    }
    return;
  }
  // each thread computes four consecutive phase steps of one (phase, 4
  // channels) with a sliding window of input rows in registers: per tap one
  // weight and one new input row are read from LDS for 16 FMAs
  const int items = (p.TJ / 4) * per_row;  // TJ is a multiple of 4
  for (int e = threadIdx.x; e < items; e += 256) {
    const int jg = e / per_row, rem = e - jg * per_row;
    const int pl = rem / p.CV, v = rem - pl * p.CV;
    const int r = r0 + pl, jl0 = 4 * jg;
    if (r >= p.R || c40 + v >= p.C4) continue;
    const float4* xr = xs + (size_t)jl0 * per_row + pl * p.CV + v;
    float4 acc[4], win[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    win[0] = xr[0];
    win[1] = xr[per_row];
    win[2] = xr[2 * per_row];
#pragma unroll 4
    for (int k = 0; k < p.K; ++k) {
      win[3] = xr[(size_t)(k + 3) * per_row];  // row jl0 + k + 3 <= TJ + K - 2
      const float4 wv = ws[k * p.CV + v];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[u].x = __builtin_fmaf(wv.x, win[u].x, acc[u].x);
        acc[u].y = __builtin_fmaf(wv.y, win[u].y, acc[u].y);
        acc[u].z = __builtin_fmaf(wv.z, win[u].z, acc[u].z);
        acc[u].w = __builtin_fmaf(wv.w, win[u].w, acc[u].w);
      }
      win[0] = win[1];
      win[1] = win[2];
      win[2] = win[3];
    }
    const int n_r = (p.T - r + p.d - 1) / p.d;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + jl0 + u;
      if (j < n_r) p.y[yb + ((size_t)r + (size_t)p.d * j) * p.C4 + c40 + v] = acc[u];
    }
  }
}

// Tile choice: up to 64 phase steps, then as many phases as keep about 64
// output rows per workgroup, halved until the staged rows and weights fit in
// 64 KB (two or more workgroups per CU).
void dwconv1d_tile(int T, int C, int K, int d, int* tj, int* pp, int* cv, int* lds) {
  const int R = d < T ? d : T;
  const int n_max = (T + d - 1) / d;
  int TJ = n_max < 64 ? n_max : 64;
  TJ = (TJ + 3) / 4 * 4;  // whole groups of four phase steps per thread
  int P = 64 / TJ;
  if (P < 1) P = 1;
  if (P > R) P = R > 0 ? R : 1;
  const int CV = C / 4 < 16 ? C / 4 : 16;
  auto bytes = [&](int tjv, int pv) { return ((tjv + K - 1) * pv + K) * CV * 16; };
  while (bytes(TJ, P) > 65536 && (P > 1 || TJ > 4)) {
    if (P > 1) P /= 2;
    else TJ = (TJ / 2 + 3) / 4 * 4;
  }
  *tj = TJ; *pp = P; *cv = CV; *lds = bytes(TJ, P);
}

hipError_t launch_dwconv1d(const float* x, const float* w, float* y, int B, int T, int C, int K, int d,
                           hipStream_t st) {
  DwParams p;
  p.x = (const float4*)x; p.w = (const float4*)w; p.y = (float4*)y;
  p.B = B; p.T = T; p.C4 = C / 4; p.K = K; p.d = d;
  p.L = T + d * (K - 1);
  p.R = d < T ? d : T;
  int lds = 0;
  dwconv1d_tile(T, C, K, d, &p.TJ, &p.P, &p.CV, &lds);
  p.pgroups = (p.R + p.P - 1) / p.P;
  p.jtiles = ((T + d - 1) / d + p.TJ - 1) / p.TJ;
  p.cchunks = (p.C4 + p.CV - 1) / p.CV;
  p.four = (p.TJ / 4) * p.P * p.CV >= 256 ? 1 : 0;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const size_t grid = (size_t)B * p.pgroups * p.jtiles * p.cchunks;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)k_dwconv1d, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  DEFT_LAUNCH("dwconv1d", k_dwconv1d, dim3((unsigned)grid), dim3(256), lds, st, p);
  return hipGetLastError();
}

}  // namespace deft
