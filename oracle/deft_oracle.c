/*
 * deft_oracle.c -- CPU oracle for the deformable 3x3 convolution layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under irregular_gather_cnn_amd/csrc) shares no code with it and
 * never calls it.
 *
 * What it computes follows the DefT explainer page ("DefT: Boosting
 * Scalability of Deformable Convolution Operations on GPUs"): a deformable
 * layer is three operators run back to back (section "The argument in one
 * glance", part "What people did"): an offset convolution over the same input
 * that yields a fractional offset for every filter position at every output
 * location ("Following a deformable layer through DefT", step 1), a bilinear
 * interpolation that gathers the four neighbours around each displaced sample
 * and blends them by weight ("Why it fell short"), and the main convolution
 * over the resulting deformed column buffer.  The page prints no formula; the
 * plainest reading (deformable convolution v1, no modulation) is written out
 * below as O1..O5, and the backward pass B1..B6 is the exact derivative of it
 * (the page only mentions training time).
 *
 * Arithmetic is fp64 (inputs arrive already upcast, exactly, from fp32 or
 * bf16).  Loops are the definitions written out; OpenMP splits independent
 * output elements only, so every output's summation order is the one written.
 * Integer decisions are the exception: which cell of four neighbours a
 * sample point falls in, and whether it is fully outside, are taken on the
 * fp32 coordinate (the fp32 offset added to the integer grid position in one
 * fp32 add), the precision the layer hands offsets over in; see
 * sample_point and oracle_sample_index_f32.  The value is continuous across
 * a cell edge, but its derivative in the offset is not, so the backward pass
 * depends on that choice.  This file must be compiled with -ffp-contract=off
 * and without -ffast-math.
 *
 * Notation: K = kh*kw taps, tap k = i*kw + j; G offset groups of Cg = Cin/G
 * channels; Oc = 2*G*K offset channels, channel 2*(g*K+k) holds dy and
 * 2*(g*K+k)+1 holds dx; Ho = floor((H + 2p - d(kh-1) - 1)/s) + 1.
 * Layouts: x [N][Cin][H][W]; w_off [Oc][Cin][kh][kw]; w [Cout][Cin][kh][kw];
 * off [N][Oc][Ho][Wo]; col [N][Ho*Wo][Cin][K] (pixel-major, channel, tap);
 * y [N][Cout][Ho][Wo].
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int n, c_in, h, w, c_out, kh, kw;
  int stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
  int groups;
} odesc;

static int out_h(const odesc* d) {
  return (d->h + 2 * d->pad_h - d->dil_h * (d->kh - 1) - 1) / d->stride_h + 1;
}
static int out_w(const odesc* d) {
  return (d->w + 2 * d->pad_w - d->dil_w * (d->kw - 1) - 1) / d->stride_w + 1;
}

/* Threads the OpenMP loops below use. */
int oracle_threads(void) { return omp_get_max_threads(); }

int oracle_out_hw(const odesc* d, int* ho, int* wo) {
  *ho = out_h(d);
  *wo = out_w(d);
  return 0;
}

/* Zero-padded read of the input: locations outside the image read 0. */
static double xz(const odesc* d, const double* x, int n, int c, int y, int xx) {
  if (y < 0 || y >= d->h || xx < 0 || xx >= d->w) return 0.0;
  return x[(((size_t)n * d->c_in + c) * d->h + y) * d->w + xx];
}

/* O1: the offset convolution, a plain linear convolution with the main
 * convolution's kernel size, stride, padding and dilation, over all input
 * channels, plus bias. */
void oracle_offset_conv(const odesc* d, const double* x, const double* w_off,
                        const double* b_off, double* off) {
  const int K = d->kh * d->kw, Oc = 2 * d->groups * K;
  const int Ho = out_h(d), Wo = out_w(d);
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < d->n; ++n)
    for (int o = 0; o < Oc; ++o)
      for (int ho = 0; ho < Ho; ++ho)
        for (int wo = 0; wo < Wo; ++wo) {
          double acc = b_off ? b_off[o] : 0.0;
          for (int c = 0; c < d->c_in; ++c)
            for (int i = 0; i < d->kh; ++i)
              for (int j = 0; j < d->kw; ++j)
                acc += w_off[(((size_t)o * d->c_in + c) * d->kh + i) * d->kw + j] *
                       xz(d, x, n, c, ho * d->stride_h - d->pad_h + i * d->dil_h,
                          wo * d->stride_w - d->pad_w + j * d->dil_w);
          off[(((size_t)n * Oc + o) * Ho + ho) * Wo + wo] = acc;
        }
}

/* O2 + O3: the sample point of tap k = (i, j) of output (ho, wo) for the
 * offset group g: the base grid position plus (dy, dx) read from offset
 * channels 2(gK+k) and 2(gK+k)+1, in fp64 (py, px).  Its cell (y0, x0) and
 * the fully-outside test are decided on the fp32 coordinate, exactly as in
 * oracle_sample_index_f32: fy = base + (float)dy in one fp32 add; fully
 * outside unless -1 < fy < H and -1 < fx < W (NaN compares false, so it is
 * outside); otherwise y0 = floor(fy), x0 = floor(fx).  Where fy rounds across
 * an integer that py does not reach, ly = py - y0 below falls outside [0, 1]
 * by less than one fp32 ulp of the coordinate. */
typedef struct {
  double py, px;
  int y0, x0, outside;
} tap_pt;

static tap_pt sample_point(const odesc* d, const double* off, int n, int g, int k, int ho,
                           int wo) {
  const int K = d->kh * d->kw, Oc = 2 * d->groups * K;
  const int Ho = out_h(d), Wo = out_w(d);
  const int i = k / d->kw, j = k % d->kw;
  const int by = ho * d->stride_h - d->pad_h + i * d->dil_h;
  const int bx = wo * d->stride_w - d->pad_w + j * d->dil_w;
  const double dy = off[(((size_t)n * Oc + 2 * (g * K + k)) * Ho + ho) * Wo + wo];
  const double dx = off[(((size_t)n * Oc + 2 * (g * K + k) + 1) * Ho + ho) * Wo + wo];
  tap_pt t;
  t.py = (double)by + dy;
  t.px = (double)bx + dx;
  const volatile float fy = (float)by + (float)dy;
  const volatile float fx = (float)bx + (float)dx;
  t.outside = !(fy > -1.0f && fy < (float)d->h && fx > -1.0f && fx < (float)d->w);
  t.y0 = t.outside ? 0 : (int)floorf(fy);
  t.x0 = t.outside ? 0 : (int)floorf(fx);
  return t;
}

/* O3 + O4 for one sample point: bilinear interpolation of channel c of image
 * n with zero padding per corner.  A fully outside point reads 0 and has zero
 * weights.  Otherwise ly = py - y0, lx = px - x0 and the value is the
 * (1-ly)(1-lx), (1-ly)lx, ly(1-lx), ly*lx weighted sum of the four corners
 * (y0,x0), (y0,x0+1), (y0+1,x0), (y0+1,x0+1). */
static double bilinear(const odesc* d, const double* x, int n, int c, tap_pt t) {
  if (t.outside) return 0.0;
  const int y0 = t.y0, x0 = t.x0;
  const double ly = t.py - y0, lx = t.px - x0;
  return (1.0 - ly) * (1.0 - lx) * xz(d, x, n, c, y0, x0) +
         (1.0 - ly) * lx * xz(d, x, n, c, y0, x0 + 1) +
         ly * (1.0 - lx) * xz(d, x, n, c, y0 + 1, x0) +
         ly * lx * xz(d, x, n, c, y0 + 1, x0 + 1);
}

/* O4 for every (n, pixel, channel, tap): the deformed column buffer. */
void oracle_sample_cols(const odesc* d, const double* x, const double* off, double* col) {
  const int K = d->kh * d->kw, Cg = d->c_in / d->groups;
  const int Ho = out_h(d), Wo = out_w(d);
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < d->n; ++n)
    for (int ho = 0; ho < Ho; ++ho)
      for (int wo = 0; wo < Wo; ++wo)
        for (int c = 0; c < d->c_in; ++c)
          for (int k = 0; k < K; ++k) {
            col[((((size_t)n * Ho + ho) * Wo + wo) * d->c_in + c) * K + k] =
                bilinear(d, x, n, c, sample_point(d, off, n, c / Cg, k, ho, wo));
          }
}

/* O5: the main convolution over the deformed columns, plus bias. */
void oracle_main_conv(const odesc* d, const double* col, const double* w, const double* b,
                      double* y) {
  const int K = d->kh * d->kw, Ck = d->c_in * K;
  const int Ho = out_h(d), Wo = out_w(d);
  const size_t P = (size_t)Ho * Wo;
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < d->n; ++n)
    for (int co = 0; co < d->c_out; ++co)
      for (size_t p = 0; p < P; ++p) {
        const double* cr = col + ((size_t)n * P + p) * Ck;
        const double* wr = w + (size_t)co * Ck;
        double acc = b ? b[co] : 0.0;
        for (int e = 0; e < Ck; ++e) acc += wr[e] * cr[e];
        y[((size_t)n * d->c_out + co) * P + p] = acc;
      }
}

/* The whole forward pass.  off_out and col_out may be NULL; col_out, when
 * given, receives the deformed columns [N][Ho*Wo][Cin][K]. */
void oracle_forward(const odesc* d, const double* x, const double* w_off, const double* b_off,
                    const double* w, const double* b, double* y, double* off_out,
                    double* col_out) {
  const int K = d->kh * d->kw, Oc = 2 * d->groups * K;
  const size_t P = (size_t)out_h(d) * out_w(d);
  double* off = off_out ? off_out : (double*)malloc(sizeof(double) * d->n * Oc * P + 8);
  double* col = col_out ? col_out : (double*)malloc(sizeof(double) * d->n * P * d->c_in * K + 8);
  oracle_offset_conv(d, x, w_off, b_off, off);
  oracle_sample_cols(d, x, off, col);
  oracle_main_conv(d, col, w, b, y);
  if (!off_out) free(off);
  if (!col_out) free(col);
}

/* Backward pass, exact derivative of O1..O5.  Inputs: x, w_off, w, the
 * forward's offsets off, the upstream gradient dy [N][Cout][Ho][Wo].
 * Outputs (all required): dx [N][Cin][H][W], dw_off, db_off, dw, db, and
 * doff [N][Oc][Ho][Wo].
 *   B1  db = sum dY;  dW[co][c][k] = sum_{n,p} dY[n][co][p] col[n][p][c][k]
 *   B2  dcol[n][p][c][k] = sum_co W[co][c][k] dY[n][co][p]
 *   B3  dx_s: each in-image corner of each not-fully-outside tap receives
 *       dcol times that corner's bilinear weight
 *   B4  ddy, ddx: derivative of the bilinear value in py, px within the
 *       point's cell (y0, x0) (so one-sided at a cell edge, on the side the
 *       fp32 floor chose), summed over the channels of the tap's offset group
 *   B5  db_off = sum doff; dW_off = doff against the plain im2col of x;
 *       dx_o = transposed convolution of doff with W_off
 *   B6  dx = dx_s + dx_o */
void oracle_backward(const odesc* d, const double* x, const double* w_off, const double* w,
                     const double* off, const double* dyv, double* dx, double* dw_off,
                     double* db_off, double* dw, double* db, double* doff) {
  const int K = d->kh * d->kw, Oc = 2 * d->groups * K, Ck = d->c_in * K;
  const int Cg = d->c_in / d->groups;
  const int Ho = out_h(d), Wo = out_w(d);
  const size_t P = (size_t)Ho * Wo;
  double* col = (double*)malloc(sizeof(double) * d->n * P * Ck + 8);
  double* dcol = (double*)malloc(sizeof(double) * d->n * P * Ck + 8);
  oracle_sample_cols(d, x, off, col);

  /* B1 */
#pragma omp parallel for schedule(static)
  for (int co = 0; co < d->c_out; ++co) {
    double acc = 0.0;
    for (int n = 0; n < d->n; ++n)
      for (size_t p = 0; p < P; ++p) acc += dyv[((size_t)n * d->c_out + co) * P + p];
    db[co] = acc;
  }
#pragma omp parallel for collapse(2) schedule(static)
  for (int co = 0; co < d->c_out; ++co)
    for (int e = 0; e < Ck; ++e) {
      double acc = 0.0;
      for (int n = 0; n < d->n; ++n)
        for (size_t p = 0; p < P; ++p)
          acc += dyv[((size_t)n * d->c_out + co) * P + p] * col[((size_t)n * P + p) * Ck + e];
      dw[(size_t)co * Ck + e] = acc;
    }

  /* B2 */
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < d->n; ++n)
    for (size_t p = 0; p < P; ++p)
      for (int e = 0; e < Ck; ++e) {
        double acc = 0.0;
        for (int co = 0; co < d->c_out; ++co)
          acc += w[(size_t)co * Ck + e] * dyv[((size_t)n * d->c_out + co) * P + p];
        dcol[((size_t)n * P + p) * Ck + e] = acc;
      }

  /* B3: scatter into dx, one (n, c) plane per thread so there is no race. */
  memset(dx, 0, sizeof(double) * d->n * d->c_in * d->h * d->w);
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < d->n; ++n)
    for (int c = 0; c < d->c_in; ++c) {
      double* plane = dx + ((size_t)n * d->c_in + c) * d->h * d->w;
      for (int ho = 0; ho < Ho; ++ho)
        for (int wo = 0; wo < Wo; ++wo)
          for (int k = 0; k < K; ++k) {
            const tap_pt t = sample_point(d, off, n, c / Cg, k, ho, wo);
            if (t.outside) continue;
            const double g = dcol[(((size_t)n * P + (size_t)ho * Wo + wo) * d->c_in + c) * K + k];
            const int y0 = t.y0, x0 = t.x0;
            const double ly = t.py - y0, lx = t.px - x0;
            const int cy[4] = {y0, y0, y0 + 1, y0 + 1};
            const int cx[4] = {x0, x0 + 1, x0, x0 + 1};
            const double cw[4] = {(1.0 - ly) * (1.0 - lx), (1.0 - ly) * lx, ly * (1.0 - lx),
                                  ly * lx};
            for (int q = 0; q < 4; ++q)
              if (cy[q] >= 0 && cy[q] < d->h && cx[q] >= 0 && cx[q] < d->w)
                plane[(size_t)cy[q] * d->w + cx[q]] += g * cw[q];
          }
    }

  /* B4 */
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < d->n; ++n)
    for (int g = 0; g < d->groups; ++g)
      for (int k = 0; k < K; ++k)
        for (int ho = 0; ho < Ho; ++ho)
          for (int wo = 0; wo < Wo; ++wo) {
            double gy = 0.0, gx = 0.0;
            const tap_pt t = sample_point(d, off, n, g, k, ho, wo);
            if (!t.outside) {
              const int y0 = t.y0, x0 = t.x0;
              const double ly = t.py - y0, lx = t.px - x0;
              for (int c = g * Cg; c < (g + 1) * Cg; ++c) {
                const double v00 = xz(d, x, n, c, y0, x0), v01 = xz(d, x, n, c, y0, x0 + 1);
                const double v10 = xz(d, x, n, c, y0 + 1, x0), v11 = xz(d, x, n, c, y0 + 1, x0 + 1);
                const double gc =
                    dcol[(((size_t)n * P + (size_t)ho * Wo + wo) * d->c_in + c) * K + k];
                gy += gc * ((1.0 - lx) * (v10 - v00) + lx * (v11 - v01));
                gx += gc * ((1.0 - ly) * (v01 - v00) + ly * (v11 - v10));
              }
            }
            doff[(((size_t)n * Oc + 2 * (g * K + k)) * Ho + ho) * Wo + wo] = gy;
            doff[(((size_t)n * Oc + 2 * (g * K + k) + 1) * Ho + ho) * Wo + wo] = gx;
          }

  /* B5 */
  for (int o = 0; o < Oc; ++o) {
    double acc = 0.0;
    for (int n = 0; n < d->n; ++n)
      for (size_t p = 0; p < P; ++p) acc += doff[((size_t)n * Oc + o) * P + p];
    db_off[o] = acc;
  }
#pragma omp parallel for collapse(2) schedule(static)
  for (int o = 0; o < Oc; ++o)
    for (int c = 0; c < d->c_in; ++c)
      for (int i = 0; i < d->kh; ++i)
        for (int j = 0; j < d->kw; ++j) {
          double acc = 0.0;
          for (int n = 0; n < d->n; ++n)
            for (int ho = 0; ho < Ho; ++ho)
              for (int wo = 0; wo < Wo; ++wo)
                acc += doff[(((size_t)n * Oc + o) * Ho + ho) * Wo + wo] *
                       xz(d, x, n, c, ho * d->stride_h - d->pad_h + i * d->dil_h,
                          wo * d->stride_w - d->pad_w + j * d->dil_w);
          dw_off[(((size_t)o * d->c_in + c) * d->kh + i) * d->kw + j] = acc;
        }
  /* dx_o: every (n, c) plane gathers the transposed convolution. */
#pragma omp parallel for collapse(2) schedule(static)
  for (int n = 0; n < d->n; ++n)
    for (int c = 0; c < d->c_in; ++c) {
      double* plane = dx + ((size_t)n * d->c_in + c) * d->h * d->w;
      for (int o = 0; o < Oc; ++o)
        for (int i = 0; i < d->kh; ++i)
          for (int j = 0; j < d->kw; ++j) {
            const double wv = w_off[(((size_t)o * d->c_in + c) * d->kh + i) * d->kw + j];
            for (int ho = 0; ho < Ho; ++ho)
              for (int wo = 0; wo < Wo; ++wo) {
                const int yy = ho * d->stride_h - d->pad_h + i * d->dil_h;
                const int xx = wo * d->stride_w - d->pad_w + j * d->dil_w;
                if (yy < 0 || yy >= d->h || xx < 0 || xx >= d->w) continue;
                plane[(size_t)yy * d->w + xx] +=
                    wv * doff[(((size_t)n * Oc + o) * Ho + ho) * Wo + wo];
              }
          }
    }
  free(col);
  free(dcol);
}

/* The integer tap-index / corner-mask stage, defined in fp32.  For each
 * (n, g, k, ho, wo), from the fp32 offsets:
 *   base = ho*s - p + i*d (int32, converted to float exactly)
 *   py = base + dy (one fp32 add, round to nearest even), px likewise
 *   fully outside unless -1 < py < H and -1 < px < W, compared in fp32;
 *   then y0 = x0 = 0 and mask = 0
 *   otherwise y0 = floor(py), x0 = floor(px); mask bit q is set when corner
 *   q lies in the image, corners ordered (y0,x0), (y0,x0+1), (y0+1,x0),
 *   (y0+1,x0+1).
 * Outputs are laid out [N][G][K][Ho][Wo]. */
void oracle_sample_index_f32(const odesc* d, const float* off, int32_t* y0o, int32_t* x0o,
                             uint8_t* mask) {
  const int K = d->kh * d->kw, Oc = 2 * d->groups * K;
  const int Ho = out_h(d), Wo = out_w(d);
  for (int n = 0; n < d->n; ++n)
    for (int g = 0; g < d->groups; ++g)
      for (int k = 0; k < K; ++k)
        for (int ho = 0; ho < Ho; ++ho)
          for (int wo = 0; wo < Wo; ++wo) {
            const int i = k / d->kw, j = k % d->kw;
            const float dy = off[(((size_t)n * Oc + 2 * (g * K + k)) * Ho + ho) * Wo + wo];
            const float dx = off[(((size_t)n * Oc + 2 * (g * K + k) + 1) * Ho + ho) * Wo + wo];
            const volatile float py = (float)(ho * d->stride_h - d->pad_h + i * d->dil_h) + dy;
            const volatile float px = (float)(wo * d->stride_w - d->pad_w + j * d->dil_w) + dx;
            const size_t o = ((((size_t)n * d->groups + g) * K + k) * Ho + ho) * Wo + wo;
            if (!(py > -1.0f && py < (float)d->h && px > -1.0f && px < (float)d->w)) {
              y0o[o] = 0;
              x0o[o] = 0;
              mask[o] = 0;
              continue;
            }
            const int y0 = (int)floorf(py), x0 = (int)floorf(px);
            uint8_t m = 0;
            if (y0 >= 0 && x0 >= 0) m |= 1;
            if (y0 >= 0 && x0 + 1 < d->w) m |= 2;
            if (y0 + 1 < d->h && x0 >= 0) m |= 4;
            if (y0 + 1 < d->h && x0 + 1 < d->w) m |= 8;
            y0o[o] = y0;
            x0o[o] = x0;
            mask[o] = m;
          }
}
