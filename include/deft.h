/*
 * deft.h -- C ABI of the MI355X (gfx950) deformable 3x3 convolution library.
 *
 * The layer (DefT explainer page, "The argument in one glance", parts "What
 * people did" and "This paper's idea"; "Following a deformable layer through
 * DefT", step 1): an offset convolution over the input predicts, for every
 * filter tap at every output pixel, a fractional (dy, dx); each tap's sample
 * point (its grid position plus that offset) is bilinearly interpolated from
 * its four neighbouring input pixels into a deformed column buffer; the main
 * convolution is a dense GEMM over those columns.  The offset convolution and
 * the sampling run fused in one kernel so the offsets never leave the chip,
 * and the input tile plus a halo sized from the offset distribution is staged
 * in LDS (section "How DefT works", "The idea"; "Why it works").
 *
 * Conventions for every call:
 *  - Tensors are dense, row-major, on the device, owned by the caller.  The
 *    library allocates no device memory in forward/backward; all scratch lives
 *    in the caller's workspace.
 *  - x [N][Cin][H][W]; w_off [Oc][Cin][kh][kw] with Oc = 2*G*kh*kw, channel
 *    2*(g*kh*kw + k) is dy and 2*(g*kh*kw + k)+1 is dx of tap k = i*kw + j of
 *    offset group g (channels [g*Cin/G, (g+1)*Cin/G)); b_off [Oc];
 *    w [Cout][Cin][kh][kw]; b [Cout]; y [N][Cout][Ho][Wo];
 *    offsets [N][Oc][Ho][Wo] are always fp32.  x, weights, biases, y, dy and
 *    the gradients have the descriptor's dtype.
 *  - Ho = (H + 2*pad_h - dil_h*(kh-1) - 1)/stride_h + 1, likewise Wo.
 *  - Out-of-image corners read zero; a tap whose sample point is not inside
 *    -1 < py < H, -1 < px < W (or is NaN) reads zero and gets no gradient.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous on that stream; nothing synchronises implicitly.
 *  - Return 0 on success or a negative DEFT_ERR_* code.  Every argument is
 *    validated before anything is launched; on error nothing is launched and
 *    no output is touched.  A plan with N = 0 makes deft_forward,
 *    deft_backward and deft_debug_sample no-ops that return 0 without
 *    checking the tensor pointers (an empty batch has none).
 */
#ifndef DEFT_H
#define DEFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum deft_dtype { DEFT_F32 = 0, DEFT_BF16 = 1 };

enum deft_status {
  DEFT_OK = 0,
  DEFT_ERR_BAD_DESC = -1,     /* non-positive size, kernel, stride or dilation; negative pad */
  DEFT_ERR_GROUPS = -2,       /* offset_groups < 1 or Cin not divisible by it */
  DEFT_ERR_SHAPE = -3,        /* Ho or Wo < 1 */
  DEFT_ERR_NULLPTR = -4,      /* a required pointer is NULL */
  DEFT_ERR_WORKSPACE = -5,    /* workspace NULL or smaller than deft_workspace_bytes */
  DEFT_ERR_DTYPE = -6,        /* dtype not DEFT_F32 / DEFT_BF16 */
  DEFT_ERR_ALIGN = -7,        /* a device pointer is not 16-byte aligned */
  DEFT_ERR_HIP = -8,          /* a HIP runtime call or launch failed */
  DEFT_ERR_PLAN = -9,         /* forced tile/halo/chunk outside the supported range */
  DEFT_ERR_UNSUPPORTED = -10, /* channels per offset group not a multiple of 16, or size limits */
  DEFT_ERR_SCRATCH = -11      /* deft_forward_noalloc: the plan's forward scratch exceeds
                                 DEFT_NOALLOC_SCRATCH_BYTES */
};

/* Size of the static device scratch of deft_forward_noalloc (per GPU). */
#define DEFT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Layer descriptor.  Main-convolution groups are 1; offset_groups = G. */
typedef struct deft_desc {
  int n, c_in, h, w, c_out, kh, kw;
  int stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
  int offset_groups;
  int dtype; /* enum deft_dtype */
} deft_desc;

/* Execution plan (opaque): output tile, halo, channel chunk, launch shape. */
typedef struct deft_plan deft_plan;

typedef struct deft_plan_info {
  int tile_h, tile_w;     /* output pixels per workgroup tile of the fused kernel */
  int halo;               /* LDS halo in input pixels around the tile's footprint (LDS-halo
                             forward; unused by the direct gather) */
  int chunk;              /* channels staged per LDS pass */
  int groups_per_wg;      /* offset groups handled by one workgroup */
  int num_workgroups;     /* fused-kernel grid size */
  int ho, wo, oc;
  int lds_bytes;          /* fused-kernel LDS per workgroup */
  double est_miss_fraction; /* planner's estimate of the share of taps outside bwd_halo, which
                               take the backward's slow path (-1: forced plan) */
  size_t ws_forward, ws_training;
  size_t ws_cols_offset;  /* byte offset in the workspace of the deformed columns
                             [N*Ho*Wo][kh*kw][Cin] that deft_forward leaves there */
  int bwd_tile_h, bwd_tile_w; /* output tile of the sampling backward */
  int bwd_chunk;          /* its channel chunk; 0: this plan has no backward (LDS) */
  int gemm_direct;        /* 1: the three GEMMs stage operands with direct global-to-LDS
                             loads (bf16, Ho*Wo and c_out multiples of 8, operands under
                             2 GiB); 0: register-staged generic GEMM */
  int dw_splits;          /* pixel ranges the dW GEMM is split into (one fp32 partial each) */
  int gather_direct;      /* 1: the forward gathers corners from a channel-minor copy of x held
                             in the caches (no LDS halo; halo then bounds only the backward's
                             candidate window); 0: LDS tile + halo */
  int gather_gemm;        /* 1: the forward runs the offset conv, then one launch that gathers the
                             columns straight into the main GEMM's LDS tiles (y and the columns
                             written; the GEMM reads no columns from HBM) */
  int bwd_halo;           /* the sampling backward's candidate window: taps whose corner lies
                             within it of their grid position are scattered through LDS, the
                             others one by one with global atomics */
} deft_plan_info;

/* Checks the descriptor alone.  Pure host function. */
int deft_desc_validate(const deft_desc* d);

/* Builds a plan.  halo_hist (host memory, may be NULL) is the required-halo
 * histogram of deft_halo_histogram: hist[i] for i < hist_len-2 counts taps
 * whose corner (y0, x0) lies exactly i pixels (Chebyshev distance) from the
 * tap's grid position, hist[hist_len-2] counts taps at hist_len-2 or more,
 * hist[hist_len-1] counts fully outside taps.  The forward's LDS halo, tile
 * and chunk come from a cost estimate (columns written, input staged, taps
 * outside the halo read from the caches, LDS occupancy and launch shape);
 * the backward's halo is the smallest that leaves at most 1e-5 of the taps
 * outside it besides those in the open-ended bin hist[hist_len-2], at most
 * 16.  NULL: forward halo from default shares, backward halo 4.  (DefT
 * page, "How DefT works", "The idea": pad each tile by just enough margin
 * that most sampled pixels stay on chip; "What it costs": tile sizing
 * depends on platform and layer shape.)  A forced plan uses its halo for
 * both.  Pure host function. */
int deft_plan_create(const deft_desc* d, const uint32_t* halo_hist, int hist_len,
                     deft_plan** out);

/* Plan with a forced tile (tile_h*tile_w <= 64), halo (0..32) and channel
 * chunk (multiple of 16 dividing Cin/G, at most 64; 0 = largest that fits;
 * -1 = direct gather: the forward reads the corners from a channel-minor copy
 * of x instead of an LDS halo; Cin a multiple of 16, at most 9 taps, and
 * Cin/(vG) a power of two <= 256 with v = 8 (bf16) or 4 (fp32) channels per
 * 16 bytes; -2 = direct gather fused into the main GEMM (bf16), which also needs Cin/G and
 * Cin multiples of 32, Ho*Wo and c_out multiples of 8).
 * DEFT_ERR_PLAN if its LDS does not fit or the direct gather is unsupported; deft_backward returns DEFT_ERR_PLAN
 * for a forced plan whose backward tile does not fit even with 8 channels.
 * Forward results (offsets, columns, y) are bit-identical across plans; the
 * backward's atomically accumulated sums (dx, dw, dw_off) and the per-chunk
 * offset-gradient partials agree across plans within rounding. */
int deft_plan_create_forced(const deft_desc* d, int tile_h, int tile_w, int halo, int chunk,
                            deft_plan** out);

int deft_plan_get_info(const deft_plan* p, deft_plan_info* info);
void deft_plan_destroy(deft_plan* p);

/* Workspace bytes for deft_forward (training = 0) or for a forward whose
 * columns are kept for deft_backward (training = 1). */
size_t deft_workspace_bytes(const deft_plan* p, int training);

/* Forward of the layer (DefT explainer page, "Following a deformable layer
 * through DefT": the offset convolution predicts each tap's fractional
 * displacement, the four neighbours of every displaced tap are blended
 * bilinearly into the deformed columns, and the main convolution multiplies
 * them; "This paper's idea": the offset convolution and the interpolation run
 * as one kernel, so the offsets stay on chip).  x, w_off, w, y and workspace
 * are required; b_off and b may be NULL (zero bias).  offsets_out (fp32
 * [N][Oc][Ho][Wo]) may be NULL; when given, the fused kernel also writes the
 * offsets it computed there (needed by deft_backward).  The deformed columns
 * are left in the workspace.  DEFT_ERR_NULLPTR, DEFT_ERR_WORKSPACE (NULL or
 * smaller than deft_workspace_bytes(p, 0)), DEFT_ERR_ALIGN; checks run before
 * any launch. */
int deft_forward(const deft_plan* p, const void* x, const void* w_off, const void* b_off,
                 const void* w, const void* b, void* y, float* offsets_out, void* workspace,
                 size_t ws_bytes, void* stream);

/* deft_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * same arguments, checks, kernels and results as deft_forward, but with no
 * workspace argument.  The scratch that deft_forward takes from the workspace
 * lives in a static device array of the library, DEFT_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, which every GPU the library runs on holds until the
 * process ends.  The call allocates nothing: on the first call with a device
 * current it looks up that device's copy of the array (hipGetSymbolAddress)
 * and keeps the address.  `stream` must belong to the current device.
 * DEFT_ERR_SCRATCH, before anything is launched, when
 * deft_workspace_bytes(p, 0) exceeds DEFT_NOALLOC_SCRATCH_BYTES (at C = 256,
 * 56 x 56, bf16 that is about 16.4 MB per image: up to 3 images).  Every
 * call on one GPU shares that GPU's array and leaves its contents there
 * (the next call overwrites what it reads before reading it): calls that
 * overlap on one GPU, on different streams or threads, race and must be
 * serialised by the caller.  The columns it leaves in the array are not
 * available to deft_backward (inference only). */
int deft_forward_noalloc(const deft_plan* p, const void* x, const void* w_off, const void* b_off,
                         const void* w, const void* b, void* y, float* offsets_out, void* stream);

/* deft_forward that also observes the offset distribution: the fused
 * sampling launch adds the required-halo histogram of every tap it samples to
 * `hist` (device uint32 [hist_len], 3 <= hist_len <= 64; the same bins as
 * deft_halo_histogram).  The counts are ADDED: the caller zeroes the buffer
 * and may let several calls accumulate before re-planning with
 * deft_plan_create (DefT page, "What to keep in mind": the gains rest on the
 * offset distribution, which shifts as training goes on and differs per
 * layer).  Other outputs are those of deft_forward.  DEFT_ERR_BAD_DESC for
 * hist_len out of range, DEFT_ERR_NULLPTR for a NULL hist (N > 0),
 * DEFT_ERR_ALIGN if hist is not 4-byte aligned; checks run before any launch. */
int deft_forward_hist(const deft_plan* p, const void* x, const void* w_off, const void* b_off,
                      const void* w, const void* b, void* y, float* offsets_out, void* workspace,
                      size_t ws_bytes, uint32_t* hist, int hist_len, void* stream);

/* The same forward in the unfused three-operator form the DefT explainer page
 * compares against ("What people did before this paper", "The argument in one
 * glance"): an offset-convolution launch writes the offsets to HBM
 * (`offsets`, fp32 [N][Oc][Ho][Wo], required), a sampling launch reads them
 * back with the input and writes the deformed columns, then the GEMM.  Same
 * arguments, checks and error codes as deft_forward, plus DEFT_ERR_NULLPTR
 * when `offsets` is NULL.  y, offsets and the columns left in the workspace
 * are bit-identical to deft_forward's with the same plan (same arithmetic in
 * the same order), so deft_backward may follow it. */
int deft_forward_unfused(const deft_plan* p, const void* x, const void* w_off, const void* b_off,
                         const void* w, const void* b, void* y, float* offsets, void* workspace,
                         size_t ws_bytes, void* stream);

/* Backward of the layer.  The DefT explainer page speaks of training only
 * through its cost ("This paper's idea", "Why it works": the layer's share of
 * training time), so this is the exact derivative of deft_forward: dW and db
 * of the main convolution, dCol, the bilinear scatter of dCol into dX with the
 * offset gradient from the corner differences, and the offset convolution's
 * dW_off, db_off and its contribution to dX.  It belongs to the forward that
 * last ran on this workspace (sized with training = 1; that forward must have
 * written offsets_out, passed here as `offsets`).  dy [N][Cout][Ho][Wo].
 * Writes (overwrites) dx, dw_off, dw; db_off and db may be NULL.  Gradients
 * are accumulated in fp32 and rounded once to the dtype.  DEFT_ERR_NULLPTR,
 * DEFT_ERR_WORKSPACE, DEFT_ERR_ALIGN, DEFT_ERR_PLAN (a plan without a
 * backward: bwd_chunk 0); checks run before any launch. */
int deft_backward(const deft_plan* p, const void* x, const void* w_off, const void* w,
                  const float* offsets, const void* dy, void* workspace, size_t ws_bytes,
                  void* dx, void* dw_off, void* db_off, void* dw, void* db, void* stream);

/* The integer tap-index / corner-mask stage on its own (DefT explainer page,
 * "Following a deformable layer through DefT", step 1: every filter position
 * at every output location gets its own sampling point), from fp32 offsets:
 * for every (n, g, k, ho, wo), laid out [N][G][kh*kw][Ho][Wo]:
 * py = float(ho*s - p + i*d) + dy (one fp32 add), px likewise; fully outside
 * taps give y0 = x0 = 0, mask = 0; otherwise y0 = floor(py), x0 = floor(px)
 * and mask bit q (q = 0..3 for corners (y0,x0), (y0,x0+1), (y0+1,x0),
 * (y0+1,x0+1)) is set when that corner is in the image.  Same device code as
 * the fused kernel. */
int deft_debug_sample_index(const deft_desc* d, const float* offsets, int32_t* y0, int32_t* x0,
                            uint8_t* mask, void* stream);

/* The sampling stage alone from given fp32 offsets, as the separate
 * interpolation operator of the three-operator layer (DefT explainer page,
 * "What people did before this paper"), writing the deformed columns
 * [N][Ho*Wo][kh*kw][Cin] (tap-major, channel-minor) of the descriptor's dtype
 * to `cols`.  DEFT_ERR_NULLPTR, DEFT_ERR_ALIGN (x and cols 16-byte, offsets
 * 4-byte aligned), DEFT_ERR_PLAN; checks run before any launch. */
int deft_debug_sample(const deft_plan* p, const void* x, const float* offsets, void* cols,
                      void* stream);

/* Required-halo histogram (device uint32 [hist_len], hist_len >= 3,
 * overwritten) of fp32 offsets, as described at deft_plan_create. */
int deft_halo_histogram(const deft_desc* d, const float* offsets, uint32_t* hist, int hist_len,
                        void* stream);

/* Dilated depthwise 1-D convolution, the workload of the JAX issue page on
 * grouped and dilated convolutions (its reproduction script: depthwise
 * lax.conv_general_dilated with feature_group_count = channels, "NTC" input,
 * "TIO" kernel with one input feature per group, stride 1, VALID padding,
 * rhs_dilation = dilation).  fp32, device pointers:
 *   x [batch][steps + dilation*(ksize-1)][channels]  (channel-minor)
 *   w [ksize][channels]
 *   y [batch][steps][channels]  (written)
 *   y[b][t][c] = sum_k w[k][c] * x[b][t + k*dilation][c].
 * channels a multiple of 4, 1 <= ksize <= 256, dilation >= 1, all pointers
 * 16-byte aligned.  DEFT_ERR_BAD_DESC for sizes out of range (also when the
 * input length exceeds 2^31 - 1 steps), DEFT_ERR_NULLPTR, DEFT_ERR_ALIGN; checks
 * run before any launch.  batch = 0 or steps = 0 is a no-op.  Asynchronous on
 * `stream`; the caller owns every buffer. */
int deft_dwconv1d_forward(const float* x, const float* w, float* y, int batch, int steps, int channels,
                          int ksize, int dilation, void* stream);

/* The depthwise convolution above followed by a pointwise (1x1) convolution,
 * fused so that the depthwise result never reaches memory (the FCM abstract's
 * fused depthwise + pointwise module).  fp32, device pointers:
 *   x    [batch][steps + dilation*(ksize-1)][channels]
 *   w_dw [ksize][channels]
 *   w_pw [channels][out_channels]
 *   z    [batch][steps][out_channels]  (written)
 *   z[b][t][o] = sum_c w_pw[c][o] * sum_k w_dw[k][c] * x[b][t + k*dilation][c].
 * channels and out_channels multiples of 32, 1 <= ksize <= 256, dilation >= 1,
 * pointers 16-byte aligned; errors as for deft_dwconv1d_forward. */
int deft_dwpw1d_forward(const float* x, const float* w_dw, const float* w_pw, float* z, int batch, int steps,
                        int channels, int out_channels, int ksize, int dilation, void* stream);

/* Per-kernel timing for benchmarks (host-side events only; no device memory).
 * deft_timing_start(capacity) creates `capacity` event pairs for the calling
 * thread; while active, each kernel that deft_forward / deft_backward /
 * deft_debug_sample launch on this thread is bracketed by two events recorded
 * on the call's stream (launches beyond capacity are not recorded).
 * deft_timing_stop() waits for the last recorded event, computes each
 * launch's duration and deactivates timing; deft_timing_count and
 * deft_timing_get(i, &name, &ms) then return the i-th launch's kernel name
 * (a static string) and milliseconds.  Errors: DEFT_ERR_BAD_DESC for a
 * capacity < 1 or an index out of range, DEFT_ERR_HIP for event failures. */
int deft_timing_start(int capacity);
int deft_timing_stop(void);
int deft_timing_count(void);
int deft_timing_get(int i, const char** name, float* ms);

/* Static description of an error code. */
const char* deft_error_string(int code);

/* Text of the last HIP error seen by this thread, or "" */
const char* deft_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DEFT_H */
