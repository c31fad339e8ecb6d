// Host-side internals of the deformable convolution library: the plan and
// the launchers each kernel file exports to deft_host.cpp.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "deft.h"

struct deft_plan {
  deft_desc d;
  int cus = 256;               // compute units of the device the plan was made for
  int max_lds = 160 * 1024;    // its LDS bytes per workgroup
  int ho, wo, oc, taps, ck, cg;
  // fused sampling kernel
  int tile_h, tile_w, halo, chunk, chunk_a, gw, gsplit;
  int bhalo;                   // sampling backward's candidate window (input pixels)
  int tiles_h, tiles_w, num_tiles, num_wg, mblocks;
  int foot_h, foot_w;          // nominal tile footprint (input pixels)
  int reg_h, reg_w;            // largest halo region (input pixels)
  int pstr, pstr_a;            // LDS pixel strides (elements)
  int lds_region, lds_off, lds_info, lds_total;  // byte offsets / total
  int direct;                  // 1: corners gathered from a channel-minor copy of x (no LDS halo)
  int bwd_mf;                  // bf16 sampling backward with the scatter on the MFMA units
  int stage_d;                 // direct: footprint-staging loads per wave per channel chunk
  int oc_pad;                  // rows of the prepared offset-conv weight
  double est_miss;
  // workspace layout (byte offsets, 256-aligned)
  size_t ws_wt, ws_woff, ws_cols, ws_xh, ws_fwd_end;
  size_t ws_w2, ws_dcol, ws_dx32, ws_doff, ws_doff16, ws_wofft, ws_train_end;
  int kk_pad;                  // padded (o, tap) depth of the transposed offset conv
  // sampling backward: each workgroup owns a core tile of input pixels
  // (btile_h x btile_w) and the (output pixel, tap) pairs that touch it
  int btile_h, btile_w, btiles_h, btiles_w, num_btiles, list_cap;
  int chunk_b, lb_dx, lb_dc, lb_cnt, lb_total;
  int woff_bands;              // row bands of the offset-weight backward
  size_t ws_list, ws_lcount, ws_doffp, ws_maxbits, ws_dwpart, ws_dwoffpart, ws_biaspart;
  // bf16 GEMMs with direct global-to-LDS staging (else the generic kernel)
  int gemm_dl;
  int dw_splits, dw_kper;      // dW partials: pixel ranges of dw_kper (per image on the generic path)
  // forward with the gather fused into the main GEMM (deft_igemm.hip): the
  // offset conv writes the offsets (to the caller's buffer or ws_offs), then
  // one launch gathers, multiplies and stores y and the columns
  int igemm;
  size_t ws_offs;
};

namespace deft {

// The offset-weight backward's form with its dOffset operand in bf16 pieces
// (four workgroups per CU): bf16, at most 32 offset channels, output rows a
// multiple of 8 pixels.
inline bool woff_a16(int dtype, int oc, int wo) { return dtype == DEFT_BF16 && oc <= 32 && wo % 8 == 0; }

// Records a HIP error for deft_last_hip_error and returns DEFT_ERR_HIP.
int report_hip_error(hipError_t e);

// Timing hook (deft_timing_start): brackets a launch with events when active.
void timing_before(hipStream_t s, const char* name);
void timing_after(hipStream_t s);

#define DEFT_LAUNCH(name, kernel, grid, block, lds, stream, ...)               \
  do {                                                                        \
    ::deft::timing_before((stream), (name));                                  \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);        \
    ::deft::timing_after((stream));                                           \
  } while (0)

struct SampleArgs {
  const void* x = nullptr;
  const void* woff_p = nullptr;   // prepared offset-conv weight [oc_pad][taps][Cin]
  const void* b_off = nullptr;    // nullable, dtype
  const float* off_in = nullptr;  // sampling alone: offsets to sample from
  float* off_out = nullptr;       // nullable
  void* cols = nullptr;           // [N*Ho*Wo][taps][Cin]
  void* xh = nullptr;             // direct gather: channel-minor copy of x (workspace)
  uint32_t* hist = nullptr;       // nullable: required-halo histogram accumulated by the launch
  int hist_len = 0;
};

hipError_t launch_prep_forward(const deft_plan& p, const void* w, const void* w_off, void* wt, void* woff_p,
                               const void* x, void* xh, hipStream_t s);
// What a sampling launch computes: the fused offset conv + sampling, the
// offset conv alone (offsets to off_out), or the sampling alone from off_in.
enum SampleMode { kFusedMode = 0, kOffsetsMode = 1, kSampleMode = 2 };
hipError_t launch_sample(const deft_plan& p, SampleMode mode, const SampleArgs& a, hipStream_t s);
hipError_t launch_sample_index(const deft_desc& d, int ho, int wo, const float* off, int32_t* y0,
                               int32_t* x0, uint8_t* mask, hipStream_t s);
hipError_t launch_halo_hist(const deft_desc& d, int ho, int wo, const float* off, uint32_t* hist,
                            int hist_len, hipStream_t s);

hipError_t launch_gemm_forward(const deft_plan& p, const void* wt, const void* cols, const void* b,
                               void* y, hipStream_t s);
// dilated depthwise 1-D convolution (deft_dwconv.hip)
hipError_t launch_dwconv1d(const float* x, const float* w, float* y, int B, int T, int C, int K, int d,
                           hipStream_t st);
// fused depthwise + pointwise 1-D convolution (deft_dwpw.hip)
hipError_t launch_dwpw1d(const float* x, const float* wdw, const float* wpw, float* z, int B, int T, int C, int O,
                         int K, int d, hipStream_t st);
// gather fused into the main GEMM (deft_igemm.hip)
bool igemm_supported(const deft_plan& p);
hipError_t launch_igemm(const deft_plan& p, const void* xh, const float* off, const void* wt, const void* b,
                        void* y, void* cols, hipStream_t st);
// direct-staging bf16 GEMMs (deft_gemm_dl.hip)
bool gemm_dl_supported(const deft_plan& p);
void gemm_dl_dw_split(const deft_plan& p, int* splits, int* kper);
hipError_t dl_gemm_forward(const deft_plan& p, const void* wt, const void* cols, const void* b, void* y,
                           hipStream_t st);
hipError_t dl_gemm_dcol(const deft_plan& p, const void* w2, const void* dy, void* dcol, uint32_t* maxbits,
                        hipStream_t st);
hipError_t dl_gemm_dw(const deft_plan& p, const void* dy, const void* cols, float* part, hipStream_t st);

struct BackwardArgs {
  const void* x;
  const void* w_off;
  const void* w;
  const float* offsets;
  const void* dy;
  void* dx;
  void* dw_off;
  void* db_off;
  void* dw;
  void* db;
  char* ws;
};
hipError_t launch_backward(const deft_plan& p, const BackwardArgs& a, hipStream_t s);

}  // namespace deft
