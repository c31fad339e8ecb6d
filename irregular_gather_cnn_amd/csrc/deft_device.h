// Device-side building blocks shared by the gfx950 kernels of the deformable
// convolution library: storage types, bf16 conversion, 32x32 MFMA wrappers
// and the tap-index stage.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace deft {

typedef uint16_t bf16_t;  // bf16 storage (bit pattern)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values rounded to bf16 (nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Element type traits.  VEC = elements per 16-byte chunk.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;
  static __device__ __forceinline__ float to_f32(float v) { return v; }
  static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int VEC = 8;
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Unpack a 16-byte chunk into 8 floats (bf16) / 4 floats (f32).
__device__ __forceinline__ void unpack8(const uint4 q, float* f) {
  f[0] = bf16_lo(q.x); f[1] = bf16_hi(q.x); f[2] = bf16_lo(q.y); f[3] = bf16_hi(q.y);
  f[4] = bf16_lo(q.z); f[5] = bf16_hi(q.z); f[6] = bf16_lo(q.w); f[7] = bf16_hi(q.w);
}

// One k-chunk step of a 32x32 output block.  Each lane holds one 16-byte
// chunk of A (row lane%32) and of B (column lane%32), covering the k values
// its lane half (lane/32) owns; the two operands use the same k assignment,
// so the product pairs matching k.  bf16: one 32x32x16 MFMA; f32: four
// 32x32x2 MFMAs, one per float of the chunk.
__device__ __forceinline__ void mfma_chunk(f32x16_t& acc, const uint4 a, const uint4 b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_chunk(f32x16_t& acc, const uint4 a, const uint4 b, float) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Output tile of one GEMM workgroup: rows from m0, columns from n0, k range
// [kb, ke), z = batch / split index.
struct TileCoord {
  int m0, n0, kb, ke, z;
  int me = 0x7fffffff;  // end of the rows this tile owns (row-balanced tilings)
};

// Row (within the 32x32 block) of accumulator register r of lane `lane`;
// the column is lane % 32.
__device__ __forceinline__ int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Tap-index stage (fp32).  base_y/base_x: the tap's grid position
// (ho*s - p + i*d, exact integers).  py = base + dy is one fp32 add.  A tap
// is fully outside unless -1 < py < H and -1 < px < W (NaN is outside).
struct TapIndex {
  int y0, x0;
  float ly, lx;
  bool outside;
};
__device__ __forceinline__ TapIndex tap_index(int base_y, int base_x, float dy, float dx, int H, int W) {
  TapIndex t;
  const float py = __fadd_rn((float)base_y, dy);
  const float px = __fadd_rn((float)base_x, dx);
  t.outside = !(py > -1.0f && py < (float)H && px > -1.0f && px < (float)W);
  if (t.outside) {
    t.y0 = 0; t.x0 = 0; t.ly = 0.f; t.lx = 0.f;
  } else {
    const float fy = floorf(py), fx = floorf(px);
    t.y0 = (int)fy; t.x0 = (int)fx;
    t.ly = __fsub_rn(py, fy); t.lx = __fsub_rn(px, fx);
  }
  return t;
}
__device__ __forceinline__ uint32_t corner_mask(const TapIndex& t, int H, int W) {
  if (t.outside) return 0u;
  uint32_t m = 0;
  if (t.y0 >= 0 && t.x0 >= 0) m |= 1u;
  if (t.y0 >= 0 && t.x0 + 1 < W) m |= 2u;
  if (t.y0 + 1 < H && t.x0 >= 0) m |= 4u;
  if (t.y0 + 1 < H && t.x0 + 1 < W) m |= 8u;
  return m;
}

// Bilinear weights of corners (y0,x0), (y0,x0+1), (y0+1,x0), (y0+1,x0+1);
// all zero for a fully outside tap.
__device__ __forceinline__ void tap_weights(const TapIndex& t, float* w) {
  if (t.outside) { w[0] = w[1] = w[2] = w[3] = 0.f; return; }
  const float hy = 1.0f - t.ly, hx = 1.0f - t.lx;
  w[0] = hy * hx; w[1] = hy * t.lx; w[2] = t.ly * hx; w[3] = t.ly * t.lx;
}

// The four-corner blend in a fixed order (every path uses this one).
__device__ __forceinline__ float blend4(const float* w, float v00, float v01, float v10, float v11) {
  float a = w[0] * v00;
  a = __builtin_fmaf(w[1], v01, a);
  a = __builtin_fmaf(w[2], v10, a);
  a = __builtin_fmaf(w[3], v11, a);
  return a;
}

// XCD-aware workgroup order: gfx950 dispatches consecutive workgroup ids
// round-robin over its 8 XCDs.  This maps the hardware id to a logical id
// such that each XCD receives a contiguous range of logical ids (bijective
// for any grid size), so neighbouring tiles share that XCD's L2.
// (A build with DEFT_XCD_SWIZZLE=0 keeps the hardware order, to measure what
// the mapping does for L2 hits.)
#ifndef DEFT_XCD_SWIZZLE
#define DEFT_XCD_SWIZZLE 1
#endif
__device__ __forceinline__ int xcd_swizzle(int wg, int num_wg) {
  if (!DEFT_XCD_SWIZZLE) return wg;
  const int q = num_wg >> 3, r = num_wg & 7;
  const int xcd = wg & 7, slot = wg >> 3;
  return xcd * q + (xcd < r ? xcd : r) + slot;
}

// Division by an invariant positive integer d: q = (umulhi(x, m) + x) >> s,
// exact for 0 <= x < 2^31 (round-up multiplier method).
struct FastDiv {
  uint32_t m, s;
};
__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << 32) * ((1ull << l) - d)) / d + 1;
  return FastDiv{(uint32_t)m, l};
}
__device__ __forceinline__ int fdiv(int x, FastDiv f) {
  const uint32_t t = __umulhi((uint32_t)x, f.m);
  return (int)((t + (uint32_t)x) >> f.s);
}

template <typename T> __device__ __forceinline__ T zero_elem() { return T(0); }

// Staging of an input region into LDS as [row][col][channel] (pixel stride
// pstr elements), zero outside the image.  bf16 input with an even width is
// read as aligned 2-pixel words, 8 channels per thread, and written as two
// 16-byte channel vectors; other inputs go element by element.
struct StageGeom {
  int pairs;       // 1: 2-pixel path
  int xa;          // first (even) column of the 2-pixel grid
  int npairs;      // 2-pixel words per row
  FastDiv div;     // divides by npairs (2-pixel path) or by RW (elementwise)
};
template <typename T>
__device__ __forceinline__ StageGeom stage_geom(int W, int rx0, int RW, size_t image_elems) {
  StageGeom g;
  // 2-pixel path: bf16, even width, 32-bit offsets within one image
  g.pairs = (sizeof(T) == 2 && (W & 1) == 0 && image_elems < 0x7fffffffu) ? 1 : 0;
  g.xa = rx0 & ~1;
  g.npairs = (rx0 + RW - g.xa + 1) >> 1;
  g.div = make_fastdiv(g.pairs ? (g.npairs > 0 ? g.npairs : 1) : (RW > 0 ? RW : 1));
  return g;
}
// Channels [c0, c0+nc) (nc a multiple of 8) of image n of x [N][Cin][H][W],
// rows [ry0, ry0+RH), columns [rx0, rx0+RW).  drh divides by RH.  Called by
// all 256 threads of the workgroup.
template <typename T>
__device__ __forceinline__ void stage_region(T* dst, const T* __restrict__ x, int Cin, int H, int W, int n, int c0,
                                             int nc, int ry0, int rx0, int RH, int RW, FastDiv drh,
                                             const StageGeom& g, int pstr) {
  const T* xb = x + ((size_t)n * Cin + c0) * H * W;
  if (sizeof(T) == 2 && g.pairs) {
    // items in batches of kU per thread: all loads of a batch are in flight
    // together; offsets are 32-bit within the image's channel slab
    constexpr int kU = 4;
    const uint32_t* xw = (const uint32_t*)xb;
    const int hw2 = (H * W) >> 1;
    const int total = (nc >> 3) * RH * g.npairs;
    for (int e0 = threadIdx.x; e0 < total; e0 += 256 * kU) {
      uint32_t w[kU][8];
      int dofs[kU], rcs[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e = e0 + u * 256;
        const int ec = e < total ? e : 0;
        const int r = fdiv(ec, g.div);
        const int xp = ec - r * g.npairs;
        const int oct = fdiv(r, drh);
        const int ry = r - oct * RH;
        const int y = ry0 + ry, xx = g.xa + 2 * xp;
        const bool in = e < total && (unsigned)y < (unsigned)H && (unsigned)xx < (unsigned)W;
        const int wofs = ((oct * 8 * H + y) * W + xx) >> 1;
#pragma unroll
        for (int k = 0; k < 8; ++k) w[u][k] = in ? xw[wofs + k * hw2] : 0u;
        rcs[u] = e < total ? xx - rx0 : -2;
        dofs[u] = (ry * RW + (xx - rx0)) * pstr + oct * 8;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int rc = rcs[u];
        if (rc >= 0 && rc < RW) {
          uint4 q;
          q.x = (w[u][0] & 0xffffu) | (w[u][1] << 16); q.y = (w[u][2] & 0xffffu) | (w[u][3] << 16);
          q.z = (w[u][4] & 0xffffu) | (w[u][5] << 16); q.w = (w[u][6] & 0xffffu) | (w[u][7] << 16);
          *(uint4*)(dst + dofs[u]) = q;
        }
        if (rc + 1 >= 0 && rc + 1 < RW) {
          uint4 q;
          q.x = (w[u][0] >> 16) | (w[u][1] & 0xffff0000u); q.y = (w[u][2] >> 16) | (w[u][3] & 0xffff0000u);
          q.z = (w[u][4] >> 16) | (w[u][5] & 0xffff0000u); q.w = (w[u][6] >> 16) | (w[u][7] & 0xffff0000u);
          *(uint4*)(dst + dofs[u] + pstr) = q;
        }
      }
    }
    return;
  }
  const int total = nc * RH * RW;
  for (int e = threadIdx.x; e < total; e += 256) {
    const int r1 = fdiv(e, g.div);
    const int rx = e - r1 * RW;
    const int c = fdiv(r1, drh);
    const int ry = r1 - c * RH;
    const int y = ry0 + ry, xx = rx0 + rx;
    T v = zero_elem<T>();
    if ((unsigned)y < (unsigned)H && (unsigned)xx < (unsigned)W) v = xb[((size_t)c * H + y) * W + xx];
    dst[(ry * RW + rx) * pstr + c] = v;
  }
}

// The 2-pixel staging split into a load half (global words into registers)
// and a store half (registers into LDS), so a kernel can keep the next
// chunk's loads in flight while it computes on the current one.  A thread
// holds up to NI items (one item: 8 channels x 2 pixels).
template <int NI>
struct PairStage {
  uint32_t w[NI][8];
};
struct PairGeom {
  int ry0, rx0, RH, RW, xa, npairs, pstr, total, H, W, hw2;
  FastDiv dnp, drh;
};
// nc channels per chunk; usable when the 2-pixel path applies and the whole
// region fits the registers of one pass.
__device__ __forceinline__ PairGeom pair_geom(int H, int W, int nc, int ry0, int rx0, int RH, int RW, int pstr) {
  PairGeom g;
  g.ry0 = ry0; g.rx0 = rx0; g.RH = RH; g.RW = RW; g.pstr = pstr; g.H = H; g.W = W;
  g.xa = rx0 & ~1;
  g.npairs = (rx0 + RW - g.xa + 1) >> 1;
  g.total = RH > 0 ? (nc >> 3) * RH * g.npairs : 0;
  g.hw2 = (H * W) >> 1;
  g.dnp = make_fastdiv(g.npairs > 0 ? g.npairs : 1);
  g.drh = make_fastdiv(RH > 0 ? RH : 1);
  return g;
}
__device__ __forceinline__ void pair_item(const PairGeom& g, int e, int& oct, int& ry, int& xx) {
  const int r = fdiv(e, g.dnp);
  const int xp = e - r * g.npairs;
  oct = fdiv(r, g.drh);
  ry = r - oct * g.RH;
  xx = g.xa + 2 * xp;
}
// Buffer descriptor (gfx9 layout): 48-bit base, stride 0, `bytes` records;
// loads at offsets at or beyond it return zero.
typedef int rsrc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  rsrc_t r;
  r.x = (int)(uint32_t)a;
  r.y = (int)(uint32_t)(a >> 32);
  r.z = (int)bytes;
  r.w = 0x00020000;
  return r;
}
constexpr int kOOB = (int)0x80000000;  // buffer offset past any range: loads return zero

typedef __attribute__((address_space(3))) void lds_t;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane from the buffer straight into LDS at dst + 16*lane.
// Written as inline assembly so the compiler does not order every later LDS
// read behind these loads; completion is awaited explicitly (wait_vm).
__device__ __forceinline__ void load_lds16(const rsrc_t r, unsigned char* dst, int voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_t*)dst);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory");
}

// The same with a wave-uniform byte offset added (the buffer range check
// applies to voff + soff) and the destination given as an LDS byte address.
__device__ __forceinline__ void load_lds16_so(const rsrc_t r, uint32_t lds_addr, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_addr), "v"(voff), "s"(r),
               "s"(soff)
               : "memory");
}
// LDS byte address of a pointer into dynamic shared memory.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(const lds_t*)p);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Waits until at most n vector-memory loads of this wave are outstanding, n
// rounded down to a multiple of 4 (at most 60): waiting for more than asked
// is always safe.  n must be wave-uniform.
__device__ __forceinline__ void wait_vm_atmost(int n) {
  switch (n < 0 ? 0 : (n > 60 ? 15 : n >> 2)) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<4>(); break;
    case 2: wait_vm<8>(); break;
    case 3: wait_vm<12>(); break;
    case 4: wait_vm<16>(); break;
    case 5: wait_vm<20>(); break;
    case 6: wait_vm<24>(); break;
    case 7: wait_vm<28>(); break;
    case 8: wait_vm<32>(); break;
    case 9: wait_vm<36>(); break;
    case 10: wait_vm<40>(); break;
    case 11: wait_vm<44>(); break;
    case 12: wait_vm<48>(); break;
    case 13: wait_vm<52>(); break;
    case 14: wait_vm<56>(); break;
    default: wait_vm<60>(); break;
  }
}

// ximg: buffer over one image; c0: first channel of the chunk.  Words outside
// the image read as zero through the buffer range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_brsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
template <int NI>
__device__ __forceinline__ void pair_load(PairStage<NI>& s, const PairGeom& g, const __amdgpu_buffer_rsrc_t ximg,
                                          int c0) {
  const int plane = g.H * g.W * 2;  // bytes per channel
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int e = threadIdx.x + u * 256;
    if (e < g.total) {
      int oct, ry, xx;
      pair_item(g, e, oct, ry, xx);
      const int y = g.ry0 + ry;
      const bool in = (unsigned)y < (unsigned)g.H && (unsigned)xx < (unsigned)g.W;
      const int voff = in ? (((c0 + oct * 8) * g.H + y) * g.W + xx) * 2 : (int)0x80000000;
#pragma unroll
      for (int k = 0; k < 8; ++k) s.w[u][k] = __builtin_amdgcn_raw_buffer_load_b32(ximg, voff, k * plane, 0);
    }
  }
}
template <int NI>
__device__ __forceinline__ void pair_store(const PairStage<NI>& s, const PairGeom& g, bf16_t* dst) {
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int e = threadIdx.x + u * 256;
    if (e < g.total) {
      int oct, ry, xx;
      pair_item(g, e, oct, ry, xx);
      const int rc = xx - g.rx0;
      bf16_t* d = dst + (ry * g.RW + rc) * g.pstr + oct * 8;
      const uint32_t* w = s.w[u];
      if (rc >= 0 && rc < g.RW) {
        uint4 q;
        q.x = (w[0] & 0xffffu) | (w[1] << 16); q.y = (w[2] & 0xffffu) | (w[3] << 16);
        q.z = (w[4] & 0xffffu) | (w[5] << 16); q.w = (w[6] & 0xffffu) | (w[7] << 16);
        *(uint4*)d = q;
      }
      if (rc + 1 >= 0 && rc + 1 < g.RW) {
        uint4 q;
        q.x = (w[0] >> 16) | (w[1] & 0xffff0000u); q.y = (w[2] >> 16) | (w[3] & 0xffff0000u);
        q.z = (w[4] >> 16) | (w[5] & 0xffff0000u); q.w = (w[6] >> 16) | (w[7] & 0xffff0000u);
        *(uint4*)(d + g.pstr) = q;
      }
    }
  }
}

// 8 consecutive channels at one LDS pixel, as floats.
__device__ __forceinline__ void lds_read8(const bf16_t* src, float* f) { unpack8(*(const uint4*)src, f); }
__device__ __forceinline__ void lds_read8(const float* src, float* f) {
  const float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* src, float* f) { unpack8(*(const uint4*)src, f); }
__device__ __forceinline__ void load8(const float* src, float* f) { lds_read8(src, f); }
__device__ __forceinline__ void store8(bf16_t* dst, const float* f) {
  uint4 q;
  q.x = pack_bf16x2(f[0], f[1]); q.y = pack_bf16x2(f[2], f[3]);
  q.z = pack_bf16x2(f[4], f[5]); q.w = pack_bf16x2(f[6], f[7]);
  *(uint4*)dst = q;
}
__device__ __forceinline__ void store8(float* dst, const float* f) {
  *(float4*)dst = make_float4(f[0], f[1], f[2], f[3]);
  *(float4*)(dst + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

// 16-byte store with the non-temporal hint, for large results that a later
// kernel streams back from HBM (the deformed columns, dCol, y): they leave for
// memory at once instead of staying in the L2 and the Infinity Cache as dirty
// lines, whose write-back would otherwise compete with the next kernel's reads.
__device__ __forceinline__ void store16_nt(void* dst, const uint4 v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  v4u q;
  q.x = v.x; q.y = v.y; q.z = v.z; q.w = v.w;
  __builtin_nontemporal_store(q, (v4u*)dst);
}
__device__ __forceinline__ void store8_nt(bf16_t* dst, const float* f) {
  store16_nt(dst, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                             pack_bf16x2(f[6], f[7])));
}

}  // namespace deft
