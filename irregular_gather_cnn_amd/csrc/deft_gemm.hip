// MFMA GEMMs of the deformable convolution layer for gfx950.
//
// The main convolution is a dense contraction over the deformed columns
// (DefT explainer page, "The argument in one glance": the main convolution
// stays a GEMM, the one dense contraction of the layer), and its backward
// gives two more: dCol = W^T dY and dW = dY Col.  One kernel template serves
// all three: C[m][n] = sum_k A[m][k] B[n][k], 256 threads as 2x2 waves, each
// wave a grid of 32x32 MFMA blocks, A and B staged through a two-stage LDS
// ring whose 16-byte chunks are XOR-swizzled by row so the per-lane 16-byte
// fragment reads do not collide on banks.  A is always k-contiguous; B is
// either k-contiguous or "k-major" (contiguous along n), in which case it is
// transposed on its way into LDS (pairs of k rows packed per 32-bit word).
#include "deft_device.h"
#include "deft_internal.h"

namespace deft {

template <typename T, int BM, int BN, int KCH, class Op>
__global__ __launch_bounds__(256) void k_gemm(const Op op) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int BK = KCH * VEC;       // k elements per stage (KCH 16-byte chunks per row)
  constexpr int WM = BM / 2, WN = BN / 2, MI = WM / 32, NI = WN / 32;
  constexpr int LA = BM * KCH / 256;
  constexpr int LB = BN * KCH / 256;
  static_assert(LA >= 1 && LB >= 2 && MI >= 1 && NI >= 1 && (KCH == 4 || KCH == 8), "tile shape");
  static_assert(!Op::B_KMAJOR || (BN / VEC) % 4 == 0, "k-major B needs a multiple of 4 n-chunks");
  extern __shared__ __align__(16) unsigned char smem[];
  uint4* sA = (uint4*)smem;        // [2][BM*KCH]
  uint4* sB = sA + 2 * BM * KCH;   // [2][BN*KCH]
  const TileCoord tc = op.tile(blockIdx.x);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Row r, logical 16-byte chunk c is stored at physical chunk c ^ swz(r):
  // the 16 rows a 16-lane group reads at one chunk land on 16 distinct
  // 16-byte slots of a 256-byte bank window (and 8 rows on 8 slots of 128 B).
  auto swz = [](int r) { return (r ^ (r >> 3)) & (KCH - 1); };
  // k-major B items (VEC consecutive n at k-rows 2kp, 2kp+1): the low two
  // bits pick one of 4 n-chunks, then the k-pair, then the rest of n, so a
  // 16-lane group loads 64 contiguous bytes of 4 rows and its transposed LDS
  // stores hit 16 distinct banks.
  auto kmajor_item = [](int it, int& nc, int& kp) {
    constexpr int KP = BK / 2;
    nc = (it / (4 * KP)) * 4 + (it & 3);
    kp = (it >> 2) & (KP - 1);
  };
  auto gload = [&](int k0, uint4* ra, uint4* rb) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + i * 256, row = c / KCH, ch = c % KCH;
      ra[i] = op.load_a(tc, tc.m0 + row, k0 + ch * VEC);
    }
    if constexpr (!Op::B_KMAJOR) {
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        const int c = tid + i * 256, row = c / KCH, ch = c % KCH;
        rb[i] = op.load_b(tc, tc.n0 + row, k0 + ch * VEC);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LB / 2; ++i) {
        int nc, kp;
        kmajor_item(tid + i * 256, nc, kp);
        rb[2 * i] = op.load_bt(tc, k0 + 2 * kp, tc.n0 + nc * VEC);
        rb[2 * i + 1] = op.load_bt(tc, k0 + 2 * kp + 1, tc.n0 + nc * VEC);
      }
    }
  };
  auto sstore = [&](int s, const uint4* ra, const uint4* rb) {
    uint4* a = sA + s * BM * KCH;
    uint4* b = sB + s * BN * KCH;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = tid + i * 256, row = c / KCH, ch = c % KCH;
      a[row * KCH + (ch ^ swz(row))] = ra[i];
    }
    if constexpr (!Op::B_KMAJOR) {
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        const int c = tid + i * 256, row = c / KCH, ch = c % KCH;
        b[row * KCH + (ch ^ swz(row))] = rb[i];
      }
    } else {
      unsigned char* bb = (unsigned char*)b;
#pragma unroll
      for (int i = 0; i < LB / 2; ++i) {
        int nc, kp;
        kmajor_item(tid + i * 256, nc, kp);
        const int k = 2 * kp, ch = k / VEC, kin = k % VEC;
        const uint4 q0 = rb[2 * i], q1 = rb[2 * i + 1];
        const uint32_t w0[4] = {q0.x, q0.y, q0.z, q0.w}, w1[4] = {q1.x, q1.y, q1.z, q1.w};
        if constexpr (VEC == 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int row = nc * 8 + e;
            const uint32_t lo = (e & 1) ? (w0[e >> 1] >> 16) : (w0[e >> 1] & 0xffffu);
            const uint32_t hi = (e & 1) ? (w1[e >> 1] & 0xffff0000u) : (w1[e >> 1] << 16);
            *(uint32_t*)(bb + (row * KCH + (ch ^ swz(row))) * 16 + kin * 2) = lo | hi;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = nc * 4 + e;
            *(uint2*)(bb + (row * KCH + (ch ^ swz(row))) * 16 + kin * 4) = make_uint2(w0[e], w1[e]);
          }
        }
      }
    }
  };
  auto compute = [&](int s) {
    const uint4* a = sA + s * BM * KCH;
    const uint4* b = sB + s * BN * KCH;
#pragma unroll
    for (int ks = 0; ks < KCH / 2; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      uint4 fa[MI], fb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        fa[i] = a[row * KCH + (ch ^ swz(row))];
      }
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int row = wn * WN + j * 32 + (lane & 31);
        fb[j] = b[row * KCH + (ch ^ swz(row))];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) mfma_chunk(acc[i][j], fa[i], fb[j], T());
    }
  };

  // Two register sets: the loads for stage it+1 were issued two iterations
  // earlier, so each global load has two compute phases to land.
  const int nk = (tc.ke - tc.kb + BK - 1) / BK;
  uint4 ra0[LA], rb0[LB], ra1[LA], rb1[LB];
  auto body = [&](int it, uint4* ra, uint4* rb) {  // ra/rb hold the loads of stage it+1
    compute(it & 1);
    if (it + 1 < nk) {
      sstore((it + 1) & 1, ra, rb);
      if (it + 3 < nk) gload(tc.kb + (it + 3) * BK, ra, rb);
    }
    __syncthreads();
  };
  if (nk > 0) {
    gload(tc.kb, ra0, rb0);
    if (nk > 1) gload(tc.kb + BK, ra1, rb1);
    sstore(0, ra0, rb0);
    if (nk > 2) gload(tc.kb + 2 * BK, ra0, rb0);
    __syncthreads();
    for (int it = 0; it < nk; it += 2) {
      body(it, ra1, rb1);
      if (it + 1 < nk) body(it + 1, ra0, rb0);
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
      op.store(tc, tc.m0 + wm * WM + i * 32, tc.n0 + wn * WN + j * 32, acc[i][j], lane);
}

// 16-byte chunk of VEC elements starting at element `idx` of `base`; elements
// at positions >= lim read as zero.  `aligned` asserts idx is a multiple of
// VEC (so the chunk is 16-byte aligned).
template <typename T>
__device__ __forceinline__ uint4 load_chunk(const T* __restrict__ base, size_t idx, int valid, bool aligned) {
  constexpr int VEC = Elem<T>::VEC;
  if (valid >= VEC && aligned) return *(const uint4*)(base + idx);
  T tmp[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) tmp[e] = e < valid ? base[idx + e] : zero_elem<T>();
  return *(const uint4*)tmp;
}

// ---- forward: y[n][co][p] = b[co] + sum_e Wt[co][e] Col[n*HoWo+p][e] ----
template <typename T>
struct FwdOp {
  static constexpr bool B_KMAJOR = false;
  const T* A;     // Wt [M][K]
  const T* B;     // cols [N][K]
  const T* bias;  // nullable
  T* y;
  int M, N, K, HoWo, tilesM, tilesN, BM, BN;
  __device__ TileCoord tile(int bid) const {
    const int lb = xcd_swizzle(bid, tilesM * tilesN);
    const int nt = lb / tilesM, mt = lb - nt * tilesM;
    return TileCoord{mt * BM, nt * BN, 0, K, 0};
  }
  __device__ uint4 load_a(const TileCoord&, int m, int k) const {
    if (m >= M || k >= K) return make_uint4(0, 0, 0, 0);
    return *(const uint4*)(A + (size_t)m * K + k);
  }
  __device__ uint4 load_b(const TileCoord&, int n, int k) const {
    if (n >= N || k >= K) return make_uint4(0, 0, 0, 0);
    return *(const uint4*)(B + (size_t)n * K + k);
  }
  __device__ void store(const TileCoord&, int mb, int nb, const f32x16_t& acc, int lane) const {
    const int q = nb + (lane & 31);
    if (q >= N) return;
    const int img = q / HoWo, p = q - img * HoWo;
    T* yb = y + (size_t)img * M * HoWo + p;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mb + acc_row(lane, r);
      if (m < M) {
        const float v = acc[r] + (bias ? Elem<T>::to_f32(bias[m]) : 0.f);
        yb[(size_t)m * HoWo] = Elem<T>::from_f32(v);
      }
    }
  }
};

// ---- backward dCol: dcol[q][e] = sum_co W2[e][co] dY[n][co][p], q = n*HoWo+p ----
template <typename T>
struct DcolOp {
  static constexpr bool B_KMAJOR = true;
  const T* A;   // W2 [M=Ck][K=Cout]
  const T* dy;  // [N_img][Cout][HoWo]
  T* dcol;      // [N][M]
  uint32_t* maxbits;  // running max of |dcol| as fp32 bits (zeroed before the launch)
  int M, N, K, HoWo, tilesM, tilesN, BM, BN;
  bool vec_ok;  // HoWo % VEC == 0
  __device__ TileCoord tile(int bid) const {
    const int lb = xcd_swizzle(bid, tilesM * tilesN);
    const int nt = lb / tilesM, mt = lb - nt * tilesM;
    return TileCoord{mt * BM, nt * BN, 0, K, 0};
  }
  __device__ uint4 load_a(const TileCoord&, int m, int k) const {
    if (m >= M || k >= K) return make_uint4(0, 0, 0, 0);
    return *(const uint4*)(A + (size_t)m * K + k);
  }
  // VEC consecutive n at one k.
  __device__ uint4 load_bt(const TileCoord&, int k, int n) const {
    constexpr int VEC = Elem<T>::VEC;
    if (k >= K || n >= N) return make_uint4(0, 0, 0, 0);
    if (vec_ok && n + VEC <= N) {
      const int img = n / HoWo, p = n - img * HoWo;
      return *(const uint4*)(dy + ((size_t)img * K + k) * HoWo + p);
    }
    T tmp[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int q = n + e;
      if (q < N) {
        const int img = q / HoWo, p = q - img * HoWo;
        tmp[e] = dy[((size_t)img * K + k) * HoWo + p];
      } else {
        tmp[e] = zero_elem<T>();
      }
    }
    return *(const uint4*)tmp;
  }
  __device__ void store(const TileCoord&, int mb, int nb, const f32x16_t& acc, int lane) const {
    const int q = nb + (lane & 31);
    // max |value| of this block (valid entries only), one atomic per wave;
    // skipped when no maxbits word is given
    float mx = 0.f;
    if (maxbits && q < N) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e0 = mb + 8 * j + 4 * (lane >> 5);
        if (e0 < M)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = fabsf(acc[4 * j + r]);
            if (a <= 3.402823466e38f) mx = fmaxf(mx, a);  // NaN and Inf are flagged by the scatter instead
          }
      }
    }
    for (int s = 1; s < 64; s <<= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
    // most blocks do not raise the running max: skip their atomics
    if (maxbits && lane == 0 &&
        __float_as_uint(mx) > __hip_atomic_load(maxbits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(maxbits, __float_as_uint(mx));
    if (q >= N) return;
    T* row = dcol + (size_t)q * M;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e0 = mb + 8 * j + 4 * (lane >> 5);
      if (e0 >= M) continue;
      if constexpr (Elem<T>::VEC == 8) {
        uint2 v;
        v.x = pack_bf16x2(acc[4 * j], acc[4 * j + 1]);
        v.y = pack_bf16x2(acc[4 * j + 2], acc[4 * j + 3]);
        *(uint2*)(row + e0) = v;
      } else {
        *(float4*)(row + e0) = make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
      }
    }
  }
};

// ---- backward dW, one partial per image: dwpart[n][co][e] = sum_p dY[n][co][p] Col[n*HoWo+p][e] ----
template <typename T>
struct DwOp {
  static constexpr bool B_KMAJOR = true;
  const T* dy;    // A: [N_img][M=Cout][HoWo]
  const T* cols;  // B': [N_img*HoWo][Ck]
  float* dwpart;  // [N_img][M][Ncols]
  int M, Ncols, HoWo, tilesM, tilesN, nimg, BM, BN;
  bool vec_ok;
  __device__ TileCoord tile(int bid) const {
    const int per = tilesM * tilesN;
    const int lb = xcd_swizzle(bid, per * nimg);
    const int img = lb / per, r = lb - img * per;
    const int nt = r / tilesM, mt = r - nt * tilesM;
    return TileCoord{mt * BM, nt * BN, 0, HoWo, img};
  }
  __device__ uint4 load_a(const TileCoord& tc, int m, int k) const {
    constexpr int VEC = Elem<T>::VEC;
    if (m >= M || k >= HoWo) return make_uint4(0, 0, 0, 0);
    const size_t idx = ((size_t)tc.z * M + m) * HoWo + k;
    return load_chunk<T>(dy, idx, min(VEC, HoWo - k), vec_ok);
  }
  __device__ uint4 load_bt(const TileCoord& tc, int k, int n) const {
    if (k >= HoWo || n >= Ncols) return make_uint4(0, 0, 0, 0);
    return *(const uint4*)(cols + ((size_t)tc.z * HoWo + k) * Ncols + n);
  }
  __device__ void store(const TileCoord& tc, int mb, int nb, const f32x16_t& acc, int lane) const {
    const int n = nb + (lane & 31);
    if (n >= Ncols) return;
    float* part = dwpart + (size_t)tc.z * M * Ncols;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mb + acc_row(lane, r);
      if (m < M) part[(size_t)m * Ncols + n] = acc[r];
    }
  }
};

constexpr int kGemmKch = 8;  // 16-byte chunks per row per stage (128-byte rows)

template <typename T, int BM, int BN, class Op>
static hipError_t run_gemm(const char* name, const Op& op, int grid, hipStream_t st) {
  constexpr int lds = 2 * (BM + BN) * kGemmKch * 16;
  auto kern = k_gemm<T, BM, BN, kGemmKch, Op>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  if (grid == 0) return hipSuccess;
  DEFT_LAUNCH(name, kern, dim3(grid), dim3(256), lds, st, op);
  return hipGetLastError();
}

template <typename T>
static hipError_t gemm_forward_t(const deft_plan& p, const void* wt, const void* cols, const void* b, void* y,
                                 hipStream_t st) {
  const char* GEMM_NAME = "gemm_forward";
  FwdOp<T> op;
  op.A = (const T*)wt; op.B = (const T*)cols; op.bias = (const T*)b; op.y = (T*)y;
  op.M = p.d.c_out; op.N = p.d.n * p.ho * p.wo; op.K = p.ck; op.HoWo = p.ho * p.wo;
  op.BN = 128;
  op.tilesN = (op.N + op.BN - 1) / op.BN;
  if (op.M > 128) {
    op.BM = 256; op.tilesM = (op.M + 255) / 256;
    return run_gemm<T, 256, 128>(GEMM_NAME, op, op.tilesM * op.tilesN, st);
  } else if (op.M > 64) {
    op.BM = 128; op.tilesM = 1;
    return run_gemm<T, 128, 128>(GEMM_NAME, op, op.tilesN, st);
  }
  op.BM = 64; op.tilesM = 1;
  return run_gemm<T, 64, 128>(GEMM_NAME, op, op.tilesN, st);
}

hipError_t launch_gemm_forward(const deft_plan& p, const void* wt, const void* cols, const void* b, void* y,
                               hipStream_t st) {
  if (p.gemm_dl) return dl_gemm_forward(p, wt, cols, b, y, st);
  return p.d.dtype == DEFT_BF16 ? gemm_forward_t<bf16_t>(p, wt, cols, b, y, st)
                                : gemm_forward_t<float>(p, wt, cols, b, y, st);
}

template <typename T>
hipError_t gemm_dcol_t(const deft_plan& p, const void* w2, const void* dy, void* dcol, uint32_t* maxbits,
                       hipStream_t st) {
  const char* GEMM_NAME = "gemm_dcol";
  DcolOp<T> op;
  op.A = (const T*)w2; op.dy = (const T*)dy; op.dcol = (T*)dcol; op.maxbits = maxbits;
  op.M = p.ck; op.N = p.d.n * p.ho * p.wo; op.K = p.d.c_out; op.HoWo = p.ho * p.wo;
  op.vec_ok = (op.HoWo % Elem<T>::VEC) == 0;
  op.BM = 256; op.BN = 128;
  op.tilesM = (op.M + op.BM - 1) / op.BM;
  op.tilesN = (op.N + op.BN - 1) / op.BN;
  return run_gemm<T, 256, 128>(GEMM_NAME, op, op.tilesM * op.tilesN, st);
}

template <typename T>
hipError_t gemm_dw_t(const deft_plan& p, const void* dy, const void* cols, float* dwpart, hipStream_t st) {
  const char* GEMM_NAME = "gemm_dw";
  DwOp<T> op;
  op.dy = (const T*)dy; op.cols = (const T*)cols; op.dwpart = dwpart;
  op.M = p.d.c_out; op.Ncols = p.ck; op.HoWo = p.ho * p.wo; op.nimg = p.d.n;
  op.vec_ok = (op.HoWo % Elem<T>::VEC) == 0;
  op.BN = 128;
  op.tilesN = (op.Ncols + op.BN - 1) / op.BN;
  if (op.M > 128) {
    op.BM = 256; op.tilesM = (op.M + 255) / 256;
    return run_gemm<T, 256, 128>(GEMM_NAME, op, op.tilesM * op.tilesN * op.nimg, st);
  } else if (op.M > 64) {
    op.BM = 128; op.tilesM = 1;
    return run_gemm<T, 128, 128>(GEMM_NAME, op, op.tilesN * op.nimg, st);
  }
  op.BM = 64; op.tilesM = 1;
  return run_gemm<T, 64, 128>(GEMM_NAME, op, op.tilesN * op.nimg, st);
}

hipError_t launch_gemm_dcol(const deft_plan& p, const void* w2, const void* dy, void* dcol, uint32_t* maxbits,
                            hipStream_t st) {
  if (p.gemm_dl) return dl_gemm_dcol(p, w2, dy, dcol, maxbits, st);
  return p.d.dtype == DEFT_BF16 ? gemm_dcol_t<bf16_t>(p, w2, dy, dcol, maxbits, st)
                                : gemm_dcol_t<float>(p, w2, dy, dcol, maxbits, st);
}
hipError_t launch_gemm_dw(const deft_plan& p, const void* dy, const void* cols, float* dwpart, hipStream_t st) {
  if (p.gemm_dl) return dl_gemm_dw(p, dy, cols, dwpart, st);
  return p.d.dtype == DEFT_BF16 ? gemm_dw_t<bf16_t>(p, dy, cols, dwpart, st)
                                : gemm_dw_t<float>(p, dy, cols, dwpart, st);
}

}  // namespace deft
