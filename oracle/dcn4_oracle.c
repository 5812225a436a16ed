/*
 * dcn4_oracle.c -- plain CPU oracle for the DCNv4 forward spatial aggregation.
 *
 * TEST INFRASTRUCTURE ONLY (see dcn4_oracle.h for who may use it and for the
 * page citations).  Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math),
 * so every fp32 operation below is one IEEE operation, rounded to nearest even,
 * with subnormals kept.
 *
 * What is computed, for output pixel (n, yo, xo), group g, channel c = g*D + d:
 *
 *   y[n,yo,xo,c] = sum_{k<K} m_{g,k} * bilinear_zero_pad(x[n,:,:,c], py_k, px_k)
 *
 * with K = kh*kw points, the weights m unbounded and not normalised
 * ([DCNv4 digest] section 1), one (offset, weight) set per group shared by its
 * D = C/G channels ([DCNv4 digest] "方法1"), and the sample location
 *   standard:    p_k = base + p_grid_k + offset_scale * delta_{g,k}
 *   multi-scale: p_k = centre + s_g * (grid_k + dir_{g,k})   ([FlowDCN] 3.1)
 *
 * Readings taken where the pages are silent or their formulas were lost:
 *  R1 grid origin: sample row = yo*sh - ph + i*dh + dy, the convolution index
 *     arithmetic of [CANN Conv2D] 2.1 with padding and dilation added;
 *  R2 output size: Ho = floor((H + 2ph - dh*(kh-1) - 1)/sh) + 1 (likewise Wo);
 *  R3 tap order: k = i*kw + j, i along H (rows), j along W;
 *  R4 offset/weight row of a group: 3K values, first K interleaved pairs
 *     (dx_k, dy_k) with x along W, then the K weights m_k; groups are stored
 *     one after another per pixel: om[n,yo,xo,g,3K];
 *  R5 zero padding: a corner outside [0,H)x[0,W) contributes nothing;
 *  R6 multi-scale centre: centre = yo*sh - ph + (kh-1)/2, grid_k = i - (kh-1)/2
 *     (odd kernels, dilation 1, offset_scale 1);
 *  R7 the offset/weight tensor has the I/O dtype, scales are fp32;
 *  R13 FlowDCN's predicted scale ([FlowDCN] 3.1 splits the deformation into
 *     a predicted scale and a predicted direction, each from its own linear
 *     layer, on top of the per-group prior s_g; 3.3 bounds the scale by a
 *     per-resolution maximum Smax; the formulas were lost): the effective
 *     scale of group g at output pixel p is S = s_g * sigma[p, g], sigma an
 *     fp32 input [N, Ho, Wo, G] (whatever activation the model applies comes
 *     before it), replaced by Smax when it is larger (max_scale > 0; a NaN S
 *     stays NaN); fp32 order: S = fl(s_g * sigma), then the clamp;
 *  R14 backward (the pages give no formula; the gradient of the forward
 *     definition): at an integer location the derivative from above (the
 *     cell of the floor), a sample that is not inside has zero gradient, and
 *     the sampling decisions are the fp32 evaluation's (see dcn4o_backward);
 *  R18 DCNv3's softmax (dcn4o_softmax_weights): over the K weights of each
 *     (pixel, group) row, offsets unchanged ([DCNv4 digest] section 1);
 *  R8 fp32 evaluation order (dcn4o_forward_f32): the location is kept as an
 *     exact integer part and a fraction.  The displacement from the integer
 *     base is t = fl(offset_scale*delta) (multi-scale: t = fl(s_g * fl(grid +
 *     dir)), base = centre); f = floor(t); the fraction lh = fl(t - f); the
 *     integer part yf = base + f (exact); the sample is skipped unless
 *     -1 <= yf <= H-1 and -1 <= xf <= W-1 (NaN displacements fail the test);
 *     y0 = yf, hh = fl(1 - lh) (same for x); corner weights fl(hh*hw),
 *     fl(hh*lw), fl(lh*hw), fl(lh*lw) for (y0,x0), (y0,x0+1), (y0+1,x0),
 *     (y0+1,x0+1); coefficient fl(m*w); acc = fma(coefficient, value, acc)
 *     with k outer, corner inner, acc starting at +0; output rounded to the
 *     I/O dtype to nearest even.  (Splitting the location keeps the fraction
 *     accurate to ~1e-7 px whatever the image size; adding the offset to the
 *     absolute coordinate first would round it to the coordinate's ulp.)
 */
#include "dcn4_oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ codecs */

float dcn4o_bf16_to_f32(uint16_t h) {
  /* bf16 is the upper half of an IEEE binary32 */
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

float dcn4o_f16_to_f32(uint16_t h) {
  /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return (float)(sign ? -v : v);
}

uint16_t dcn4o_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040); /* stay a quiet NaN */
  /* round to nearest, ties to even, on the 16 bits that are dropped */
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

uint16_t dcn4o_f32_to_f16(float f) {
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  if (isnan(f)) return 0x7e00;
  double a = fabs((double)f);
  if (isinf(f) || a >= 65520.0) return sign | 0x7c00; /* overflow -> inf */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: value = q * 2^-24, q rounded half-to-even; q == 1024
     * is the smallest normal and is encoded by the same bit pattern. */
    double q = nearbyint(a * ldexp(1.0, 24));
    return sign | (uint16_t)q;
  }
  int E;
  frexp(a, &E); /* a = fr * 2^E, fr in [0.5, 1) */
  int e = E - 1; /* a in [2^e, 2^(e+1)) */
  double m = nearbyint(ldexp(a, 10 - e)); /* in [1024, 2048] */
  if (m >= 2048.0) {
    m = 1024.0;
    e += 1;
  }
  if (e + 15 >= 31) return sign | 0x7c00;
  return sign | (uint16_t)(((e + 15) << 10) | ((int)m - 1024));
}

static float load_f32(int dtype, const void* buf, int64_t i) {
  switch (dtype) {
    case DCN4O_F32: return ((const float*)buf)[i];
    case DCN4O_BF16: return dcn4o_bf16_to_f32(((const uint16_t*)buf)[i]);
    default: return dcn4o_f16_to_f32(((const uint16_t*)buf)[i]);
  }
}

static void store_io(int dtype, void* buf, int64_t i, float v) {
  switch (dtype) {
    case DCN4O_F32: ((float*)buf)[i] = v; break;
    case DCN4O_BF16: ((uint16_t*)buf)[i] = dcn4o_f32_to_bf16(v); break;
    default: ((uint16_t*)buf)[i] = dcn4o_f32_to_f16(v); break;
  }
}

static int64_t dtype_bytes(int dtype) { return dtype == DCN4O_F32 ? 4 : 2; }

/* ------------------------------------------------------------------ shapes */

int dcn4o_check(const dcn4o_shape* s, int32_t* Ho, int32_t* Wo) {
  if (!s) return -1;
  if (s->N < 0 || s->H < 1 || s->W < 1 || s->C < 1 || s->G < 1) return -1;
  if (s->C % s->G) return -1;
  if (s->kh < 1 || s->kw < 1 || s->sh < 1 || s->sw < 1) return -1;
  if (s->ph < 0 || s->pw < 0 || s->dh < 1 || s->dw < 1) return -1;
  /* keep every integer coordinate below 2^22: exact in fp32, no overflow */
  if (s->H > (1 << 20) || s->W > (1 << 20)) return -1;
  if (s->ph > (1 << 20) || s->pw > (1 << 20)) return -1;
  if (s->sh > (1 << 20) || s->sw > (1 << 20)) return -1;
  if ((int64_t)s->dh * s->kh > (1 << 20) || (int64_t)s->dw * s->kw > (1 << 20))
    return -1;
  if (s->multiscale) {
    if (!(s->kh & 1) || !(s->kw & 1)) return -1;
    if (s->dh != 1 || s->dw != 1 || s->offset_scale != 1.0f) return -1;
  }
  if (s->pixel_scales && !s->multiscale) return -1;
  if (!(s->max_scale >= 0.0f)) return -1; /* negative or NaN */
  /* R2: standard convolution output arithmetic */
  int64_t ho = ((int64_t)s->H + 2 * s->ph - (int64_t)s->dh * (s->kh - 1) - 1);
  int64_t wo = ((int64_t)s->W + 2 * s->pw - (int64_t)s->dw * (s->kw - 1) - 1);
  if (ho < 0 || wo < 0) return -1;
  ho = ho / s->sh + 1;
  wo = wo / s->sw + 1;
  if (Ho) *Ho = (int32_t)ho;
  if (Wo) *Wo = (int32_t)wo;
  return 0;
}

int64_t dcn4o_ideal_bytes(const dcn4o_shape* s, int dtype) {
  int32_t Ho, Wo;
  if (dcn4o_check(s, &Ho, &Wo)) return -1;
  int64_t K = (int64_t)s->kh * s->kw;
  int64_t in = (int64_t)s->N * s->H * s->W * s->C;
  int64_t out = (int64_t)s->N * Ho * Wo * s->C;
  int64_t om = (int64_t)s->N * Ho * Wo * s->G * 3 * K;
  int64_t b = (in + out + om) * dtype_bytes(dtype);
  if (s->multiscale) b += 4 * (int64_t)s->G;
  if (s->pixel_scales) b += 4 * (int64_t)s->N * Ho * Wo * s->G;
  return b;
}

/* ------------------------------------------------------------ the definition
 * fp64 everywhere.  bilinear_zero_pad() is the textbook bilinear sample of one
 * channel with zero outside the image (R5): four corner terms, the "factor 4"
 * of the 36HWC count ([DCNv4 digest] "GPU效率的理论分析").
 */
static double bilinear_zero_pad(const dcn4o_shape* s, int dtype, const void* x,
                                int n, int c, double py, double px) {
  double y0 = floor(py), x0 = floor(px);
  double lh = py - y0, lw = px - x0;
  double v = 0.0;
  for (int a = 0; a < 2; ++a) {
    for (int b = 0; b < 2; ++b) {
      double yy = y0 + a, xx = x0 + b;
      double w = (a ? lh : 1.0 - lh) * (b ? lw : 1.0 - lw);
      if (yy >= 0.0 && yy < s->H && xx >= 0.0 && xx < s->W) {
        int64_t idx = (((int64_t)n * s->H + (int64_t)yy) * s->W + (int64_t)xx) *
                          s->C + c;
        v += w * (double)load_f32(dtype, x, idx);
      }
    }
  }
  return v;
}

/* R13: effective scale of group g at flat output pixel p.  Without pixel
 * scales it is s_g; a clamp applies whenever max_scale > 0.  The comparison
 * is false for NaN, so a NaN scale stays NaN. */
static double scale_f64(const dcn4o_shape* s, const float* scales,
                        const float* pscales, int64_t p, int g) {
  if (!s->multiscale) return 1.0;
  double S = (double)scales[g];
  if (s->pixel_scales) S = S * (double)pscales[p * s->G + g];
  if (s->max_scale > 0.0f && S > (double)s->max_scale) S = (double)s->max_scale;
  return S;
}

static float scale_f32(const dcn4o_shape* s, const float* scales,
                       const float* pscales, int64_t p, int g) {
  if (!s->multiscale) return 1.0f;
  float S = scales[g];
  if (s->pixel_scales) S = S * pscales[p * s->G + g];
  if (s->max_scale > 0.0f && S > s->max_scale) S = s->max_scale;
  return S;
}

/* sample location of point k=(i,j) of group g at output (yo, xo), fp64 */
static void location_f64(const dcn4o_shape* s, int yo, int xo, int i, int j,
                         double dx, double dy, double sg, double* py,
                         double* px) {
  if (s->multiscale) {
    /* [FlowDCN] 3.1: centre + s_g * (grid + direction); R6 */
    int hy = (s->kh - 1) / 2, hx = (s->kw - 1) / 2;
    *py = (double)(yo * s->sh - s->ph + hy) + sg * ((double)(i - hy) + dy);
    *px = (double)(xo * s->sw - s->pw + hx) + sg * ((double)(j - hx) + dx);
  } else {
    /* R1: base of tap (i,j) plus the scaled offset */
    *py = (double)(yo * s->sh - s->ph + i * s->dh) + (double)s->offset_scale * dy;
    *px = (double)(xo * s->sw - s->pw + j * s->dw) + (double)s->offset_scale * dx;
  }
}

static int resolve_pixels(const dcn4o_shape* s, int32_t Ho, int32_t Wo,
                          const int64_t* pix, int64_t npix, int64_t* count) {
  int64_t total = (int64_t)s->N * Ho * Wo;
  if (!pix) {
    *count = total;
    return 0;
  }
  for (int64_t t = 0; t < npix; ++t)
    if (pix[t] < 0 || pix[t] >= total) return -1;
  *count = npix;
  return 0;
}

int dcn4o_forward_f64(const dcn4o_shape* s, int dtype, const void* x,
                      const void* om, const float* scales, const float* pscales,
                      double* y, const int64_t* pix, int64_t npix, int nthreads) {
  int32_t Ho, Wo;
  int64_t count;
  if (dcn4o_check(s, &Ho, &Wo)) return -1;
  if (resolve_pixels(s, Ho, Wo, pix, npix, &count)) return -1;
  const int K = s->kh * s->kw, G = s->G, C = s->C, D = C / G;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    int64_t p = pix ? pix[t] : t; /* flat output pixel (n*Ho+yo)*Wo+xo */
    int n = (int)(p / ((int64_t)Ho * Wo));
    int yo = (int)((p / Wo) % Ho);
    int xo = (int)(p % Wo);
    for (int g = 0; g < G; ++g) {
      const int64_t row = (p * G + g) * 3 * K; /* R4 */
      double sg = scale_f64(s, scales, pscales, p, g);
      for (int d = 0; d < D; ++d) {
        int c = g * D + d;
        double acc = 0.0;
        for (int i = 0; i < s->kh; ++i) {
          for (int j = 0; j < s->kw; ++j) {
            int k = i * s->kw + j; /* R3 */
            double dx = load_f32(dtype, om, row + 2 * k);
            double dy = load_f32(dtype, om, row + 2 * k + 1);
            double m = load_f32(dtype, om, row + 2 * K + k);
            double py, px;
            location_f64(s, yo, xo, i, j, dx, dy, sg, &py, &px);
            acc += m * bilinear_zero_pad(s, dtype, x, n, c, py, px);
          }
        }
        y[t * C + c] = acc;
      }
    }
  }
  return 0;
}

int dcn4o_count_terms(const dcn4o_shape* s, int dtype, const void* om,
                      const float* scales, const float* pscales,
                      int64_t* corner_terms, int64_t* inbounds_terms) {
  int32_t Ho, Wo;
  if (dcn4o_check(s, &Ho, &Wo)) return -1;
  const int K = s->kh * s->kw, G = s->G, D = s->C / G;
  int64_t terms = 0, inbounds = 0;
  /* Walk the sample points of the definition; each point of a group has four
   * corner terms for each of the group's D channels. */
  int64_t total = (int64_t)s->N * Ho * Wo;
  for (int64_t p = 0; p < total; ++p) {
    int yo = (int)((p / Wo) % Ho), xo = (int)(p % Wo);
    for (int g = 0; g < G; ++g) {
      const int64_t row = (p * G + g) * 3 * K;
      double sg = scale_f64(s, scales, pscales, p, g);
      for (int k = 0; k < K; ++k) {
        int i = k / s->kw, j = k % s->kw;
        double dx = load_f32(dtype, om, row + 2 * k);
        double dy = load_f32(dtype, om, row + 2 * k + 1);
        double py, px;
        location_f64(s, yo, xo, i, j, dx, dy, sg, &py, &px);
        double y0 = floor(py), x0 = floor(px);
        for (int a = 0; a < 2; ++a)
          for (int b = 0; b < 2; ++b) {
            double yy = y0 + a, xx = x0 + b;
            terms += D;
            if (yy >= 0.0 && yy < s->H && xx >= 0.0 && xx < s->W) inbounds += D;
          }
      }
    }
  }
  if (corner_terms) *corner_terms = terms;
  if (inbounds_terms) *inbounds_terms = inbounds;
  return 0;
}

/* ------------------------------------------------------- the fp32 evaluation
 * Same sum, every step one fp32 operation in the order R8 fixes.  The
 * geometry of one sample point is written out once here and used both by the
 * forward evaluation and by the geometry dump. */
typedef struct {
  int inside;
  int y0, x0;
  float lh, lw;
} geom_t;

static geom_t sample_geometry_f32(const dcn4o_shape* s, int yo, int xo, int i,
                                  int j, float dx, float dy, float sg) {
  float by, bx; /* exact integer base of the point */
  float ty, tx; /* displacement from the base     */
  if (s->multiscale) {
    int hy = (s->kh - 1) / 2, hx = (s->kw - 1) / 2;
    by = (float)(yo * s->sh - s->ph + hy);
    bx = (float)(xo * s->sw - s->pw + hx);
    float uy = (float)(i - hy) + dy; /* grid + direction */
    float ux = (float)(j - hx) + dx;
    ty = sg * uy; /* times the group's scale */
    tx = sg * ux;
  } else {
    by = (float)(yo * s->sh - s->ph + i * s->dh);
    bx = (float)(xo * s->sw - s->pw + j * s->dw);
    ty = s->offset_scale * dy;
    tx = s->offset_scale * dx;
  }
  float fy = floorf(ty), fx = floorf(tx);
  float yf = by + fy, xf = bx + fx; /* integers; exact while inside */
  geom_t r = {0, 0, 0, 0.0f, 0.0f};
  if (!(yf >= -1.0f && yf <= (float)(s->H - 1) && xf >= -1.0f &&
        xf <= (float)(s->W - 1)))
    return r; /* all four corners are padding (NaN displacements land here) */
  r.inside = 1;
  r.y0 = (int)yf;
  r.x0 = (int)xf;
  r.lh = ty - fy;
  r.lw = tx - fx;
  return r;
}

int dcn4o_forward_f32(const dcn4o_shape* s, int dtype, const void* x,
                      const void* om, const float* scales, const float* pscales,
                      void* y, float* acc_out, const int64_t* pix, int64_t npix,
                      int nthreads) {
  int32_t Ho, Wo;
  int64_t count;
  if (dcn4o_check(s, &Ho, &Wo)) return -1;
  if (resolve_pixels(s, Ho, Wo, pix, npix, &count)) return -1;
  const int K = s->kh * s->kw, G = s->G, C = s->C, D = C / G;
  const int H = s->H, W = s->W;
  if (nthreads < 1) nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    int64_t p = pix ? pix[t] : t;
    int n = (int)(p / ((int64_t)Ho * Wo));
    int yo = (int)((p / Wo) % Ho);
    int xo = (int)(p % Wo);
    for (int g = 0; g < G; ++g) {
      const int64_t row = (p * G + g) * 3 * K;
      float sg = scale_f32(s, scales, pscales, p, g);
      for (int d = 0; d < D; ++d) {
        int c = g * D + d;
        float acc = 0.0f;
        for (int i = 0; i < s->kh; ++i) {
          for (int j = 0; j < s->kw; ++j) {
            int k = i * s->kw + j;
            float dx = load_f32(dtype, om, row + 2 * k);
            float dy = load_f32(dtype, om, row + 2 * k + 1);
            float m = load_f32(dtype, om, row + 2 * K + k);
            geom_t q = sample_geometry_f32(s, yo, xo, i, j, dx, dy, sg);
            if (!q.inside) continue;
            float hh = 1.0f - q.lh, hw = 1.0f - q.lw;
            const int cy[4] = {q.y0, q.y0, q.y0 + 1, q.y0 + 1};
            const int cx[4] = {q.x0, q.x0 + 1, q.x0, q.x0 + 1};
            const float w[4] = {hh * hw, hh * q.lw, q.lh * hw, q.lh * q.lw};
            for (int r = 0; r < 4; ++r) {
              if (cy[r] < 0 || cy[r] >= H || cx[r] < 0 || cx[r] >= W) continue;
              int64_t idx = (((int64_t)n * H + cy[r]) * W + cx[r]) * C + c;
              float coef = m * w[r];
              acc = fmaf(coef, load_f32(dtype, x, idx), acc);
            }
          }
        }
        if (acc_out) acc_out[t * C + c] = acc;
        store_io(dtype, y, t * C + c, acc);
      }
    }
  }
  return 0;
}

int dcn4o_geometry(const dcn4o_shape* s, int dtype, const void* om,
                   const float* scales, const float* pscales, int32_t* y0,
                   int32_t* x0, float* lh, float* lw, uint8_t* inside,
                   const int64_t* pix, int64_t npix) {
  int32_t Ho, Wo;
  int64_t count;
  if (dcn4o_check(s, &Ho, &Wo)) return -1;
  if (resolve_pixels(s, Ho, Wo, pix, npix, &count)) return -1;
  const int K = s->kh * s->kw, G = s->G;
  for (int64_t t = 0; t < count; ++t) {
    int64_t p = pix ? pix[t] : t;
    int yo = (int)((p / Wo) % Ho), xo = (int)(p % Wo);
    for (int g = 0; g < G; ++g) {
      const int64_t row = (p * G + g) * 3 * K;
      float sg = scale_f32(s, scales, pscales, p, g);
      for (int k = 0; k < K; ++k) {
        int i = k / s->kw, j = k % s->kw;
        float dx = load_f32(dtype, om, row + 2 * k);
        float dy = load_f32(dtype, om, row + 2 * k + 1);
        geom_t q = sample_geometry_f32(s, yo, xo, i, j, dx, dy, sg);
        int64_t e = (t * G + g) * K + k;
        inside[e] = (uint8_t)q.inside;
        y0[e] = q.y0;
        x0[e] = q.x0;
        lh[e] = q.lh;
        lw[e] = q.lw;
      }
    }
  }
  return 0;
}

/* ----------------------------------------------------------------- backward
 * Gradients of y = sum_k m_k * B(p_k) (B the zero-padded bilinear sample of
 * one channel) for an upstream gradient gy [N,Ho,Wo,C] (reading R14):
 *   dL/dx[n,h,w,c]  = sum over the samples whose corner (h,w) lies in the
 *                     image of m_k * w_corner * gy[p,c]          (a scatter)
 *   dL/dm_k         = sum_{c in g} gy[p,c] * B_c(p_k)
 *   dL/d(dy_k)      = m_k * f * sum_{c in g} gy[p,c] * dB_c/drow
 *   dL/d(dx_k)      = m_k * f * sum_{c in g} gy[p,c] * dB_c/dcol
 * with f = offset_scale (standard) or the group's effective scale S
 * (multi-scale: the location moves by S per unit of direction), and, inside
 * the cell of corner (y0, x0) with fractions (lh, lw):
 *   dB/drow = (1-lw)(v10 - v00) + lw(v11 - v01)
 *   dB/dcol = (1-lh)(v01 - v00) + lh(v11 - v10)
 * (the derivative from above at integer locations, where B has a kink).  The
 * cell, the fractions, the inside test and S are the fp32 evaluation's
 * (sample_geometry_f32, R8/R13), so this oracle takes the same sampling
 * decisions as an fp32 implementation; every product and sum is fp64.
 * Samples that are not inside contribute nothing to any gradient.
 *
 * Also returned, for tolerance bounds: the sum of the absolute values of the
 * terms of every output (gx_abs, gom_abs) and the largest number of terms
 * of any single output (max_terms). */
int dcn4o_backward(const dcn4o_shape* s, int dtype, const void* x, const void* om,
                   const float* scales, const float* pscales, const void* gy,
                   double* gx, double* gom, double* gx_abs, double* gom_abs,
                   int64_t* max_terms) {
  int32_t Ho, Wo;
  if (dcn4o_check(s, &Ho, &Wo)) return -1;
  const int K = s->kh * s->kw, G = s->G, C = s->C, D = C / G;
  const int H = s->H, W = s->W;
  const int64_t nx = (int64_t)s->N * H * W * C;
  const int64_t npx = (int64_t)s->N * Ho * Wo;
  int32_t* gx_terms = NULL;
  if (gx) {
    memset(gx, 0, sizeof(double) * nx);
    if (gx_abs) memset(gx_abs, 0, sizeof(double) * nx);
    gx_terms = (int32_t*)calloc((size_t)nx, sizeof(int32_t));
    if (!gx_terms) return -1;
  }
  int64_t terms_max = 4 * (int64_t)D; /* every grad_om entry has 4D terms */
  for (int64_t p = 0; p < npx; ++p) {
    int n = (int)(p / ((int64_t)Ho * Wo));
    int yo = (int)((p / Wo) % Ho);
    int xo = (int)(p % Wo);
    for (int g = 0; g < G; ++g) {
      const int64_t row = (p * G + g) * 3 * K;
      const float sg = scale_f32(s, scales, pscales, p, g);
      const double f = s->multiscale ? (double)sg : (double)s->offset_scale;
      for (int k = 0; k < K; ++k) {
        int i = k / s->kw, j = k % s->kw;
        float dx = load_f32(dtype, om, row + 2 * k);
        float dy = load_f32(dtype, om, row + 2 * k + 1);
        double m = load_f32(dtype, om, row + 2 * K + k);
        geom_t q = sample_geometry_f32(s, yo, xo, i, j, dx, dy, sg);
        double gm = 0.0, gdr = 0.0, gdc = 0.0, am = 0.0, adr = 0.0, adc = 0.0;
        if (q.inside) {
          const double lh = q.lh, lw = q.lw, hh = 1.0 - lh, hw = 1.0 - lw;
          const int cy[4] = {q.y0, q.y0, q.y0 + 1, q.y0 + 1};
          const int cx[4] = {q.x0, q.x0 + 1, q.x0, q.x0 + 1};
          const double w[4] = {hh * hw, hh * lw, lh * hw, lh * lw};
          for (int d = 0; d < D; ++d) {
            const int c = g * D + d;
            const double gyc = load_f32(dtype, gy, p * C + c);
            double v[4];
            int64_t idx[4];
            for (int r = 0; r < 4; ++r) {
              int ok = cy[r] >= 0 && cy[r] < H && cx[r] >= 0 && cx[r] < W;
              idx[r] = ok ? (((int64_t)n * H + cy[r]) * W + cx[r]) * C + c : -1;
              v[r] = ok ? (double)load_f32(dtype, x, idx[r]) : 0.0;
            }
            const double B = w[0] * v[0] + w[1] * v[1] + w[2] * v[2] + w[3] * v[3];
            const double dBr = hw * (v[2] - v[0]) + lw * (v[3] - v[1]);
            const double dBc = hh * (v[1] - v[0]) + lh * (v[3] - v[2]);
            gm += gyc * B;
            gdr += gyc * dBr;
            gdc += gyc * dBc;
            am += fabs(gyc) * (w[0] * fabs(v[0]) + w[1] * fabs(v[1]) +
                               w[2] * fabs(v[2]) + w[3] * fabs(v[3]));
            adr += fabs(gyc) * (hw * (fabs(v[2]) + fabs(v[0])) + lw * (fabs(v[3]) + fabs(v[1])));
            adc += fabs(gyc) * (hh * (fabs(v[1]) + fabs(v[0])) + lh * (fabs(v[3]) + fabs(v[2])));
            if (gx) {
              for (int r = 0; r < 4; ++r) {
                if (idx[r] < 0) continue;
                const double t = m * w[r] * gyc;
                gx[idx[r]] += t;
                if (gx_abs) gx_abs[idx[r]] += fabs(t);
                gx_terms[idx[r]] += 1;
              }
            }
          }
        }
        if (gom) {
          gom[row + 2 * k] = m * f * gdc;     /* dx moves the column */
          gom[row + 2 * k + 1] = m * f * gdr; /* dy moves the row    */
          gom[row + 2 * K + k] = gm;
        }
        if (gom_abs) {
          gom_abs[row + 2 * k] = fabs(m * f) * adc;
          gom_abs[row + 2 * k + 1] = fabs(m * f) * adr;
          gom_abs[row + 2 * K + k] = am;
        }
      }
    }
  }
  if (gx) {
    for (int64_t e = 0; e < nx; ++e)
      if (gx_terms[e] > terms_max) terms_max = gx_terms[e];
    free(gx_terms);
  }
  if (max_terms) *max_terms = terms_max;
  return 0;
}

/* --------------------------------------------------- gradients of the scales
 * Group-scale mode only (reading R17).  Point k of group g at output pixel p
 * samples centre + S * u_k on each axis, u_k = fl(grid_k + d_k) the fp32
 * value the evaluation multiplies by the effective scale S (R8, R13), so
 *   dL/dS[p,g] = sum_k m_k * (u_y,k * sum_c gy * dB_c/drow
 *                            + u_x,k * sum_c gy * dB_c/dcol)
 * over the inside samples, with the cell, fractions and inside test of the
 * fp32 evaluation and fp64 arithmetic after them, as in dcn4o_backward.
 * Below the clamp S = s_g * sigma[p,g] (sigma = 1 without pixel scales):
 *   dL/dsigma[p,g] = s_g * dL/dS[p,g],  dL/ds_g = sum_p sigma[p,g] * dL/dS[p,g];
 * where the evaluation clamps (fl(s_g * sigma) > Smax) S is the constant Smax
 * and both derivatives are 0; at equality S is not clamped.  A NaN S puts no
 * sample inside: zero gradient.
 * gs, gs_abs [G] (nullable): dL/ds_g and its sum of absolute terms;
 * gp, gp_abs [N,Ho,Wo,G] (nullable; plans with pixel scales): dL/dsigma and
 * its sum of absolute terms. */
int dcn4o_backward_scales(const dcn4o_shape* s, int dtype, const void* x, const void* om,
                          const float* scales, const float* pscales, const void* gy,
                          double* gs, double* gs_abs, double* gp, double* gp_abs) {
  int32_t Ho, Wo;
  if (dcn4o_check(s, &Ho, &Wo)) return -1;
  if (!s->multiscale || (gp && !s->pixel_scales)) return -1;
  const int K = s->kh * s->kw, G = s->G, C = s->C, D = C / G;
  const int H = s->H, W = s->W;
  const int hy = (s->kh - 1) / 2, hx = (s->kw - 1) / 2;
  const int64_t npx = (int64_t)s->N * Ho * Wo;
  for (int g = 0; g < G; ++g) {
    if (gs) gs[g] = 0.0;
    if (gs_abs) gs_abs[g] = 0.0;
  }
  for (int64_t p = 0; p < npx; ++p) {
    int n = (int)(p / ((int64_t)Ho * Wo));
    int yo = (int)((p / Wo) % Ho);
    int xo = (int)(p % Wo);
    for (int g = 0; g < G; ++g) {
      const int64_t row = (p * G + g) * 3 * K;
      const float sg = scale_f32(s, scales, pscales, p, g);
      float sun = scales[g];
      if (s->pixel_scales) sun = sun * pscales[p * G + g];
      const int clamped = s->max_scale > 0.0f && sun > s->max_scale;
      const double sig = s->pixel_scales ? (double)pscales[p * G + g] : 1.0;
      double dS = 0.0, aS = 0.0;
      for (int k = 0; k < K; ++k) {
        int i = k / s->kw, j = k % s->kw;
        float dx = load_f32(dtype, om, row + 2 * k);
        float dy = load_f32(dtype, om, row + 2 * k + 1);
        double m = load_f32(dtype, om, row + 2 * K + k);
        geom_t q = sample_geometry_f32(s, yo, xo, i, j, dx, dy, sg);
        if (!q.inside) continue;
        const double uy = (float)(i - hy) + dy; /* the fp32 value grid + direction */
        const double ux = (float)(j - hx) + dx;
        const double lh = q.lh, lw = q.lw, hh = 1.0 - lh, hw = 1.0 - lw;
        const int cy[4] = {q.y0, q.y0, q.y0 + 1, q.y0 + 1};
        const int cx[4] = {q.x0, q.x0 + 1, q.x0, q.x0 + 1};
        double gdr = 0.0, gdc = 0.0, adr = 0.0, adc = 0.0;
        for (int d = 0; d < D; ++d) {
          const int c = g * D + d;
          const double gyc = load_f32(dtype, gy, p * C + c);
          double v[4];
          for (int r = 0; r < 4; ++r) {
            int ok = cy[r] >= 0 && cy[r] < H && cx[r] >= 0 && cx[r] < W;
            v[r] = ok ? (double)load_f32(dtype, x, (((int64_t)n * H + cy[r]) * W + cx[r]) * C + c)
                      : 0.0;
          }
          gdr += gyc * (hw * (v[2] - v[0]) + lw * (v[3] - v[1]));
          gdc += gyc * (hh * (v[1] - v[0]) + lh * (v[3] - v[2]));
          adr += fabs(gyc) * (hw * (fabs(v[2]) + fabs(v[0])) + lw * (fabs(v[3]) + fabs(v[1])));
          adc += fabs(gyc) * (hh * (fabs(v[1]) + fabs(v[0])) + lh * (fabs(v[3]) + fabs(v[2])));
        }
        dS += m * (uy * gdr + ux * gdc);
        aS += fabs(m) * (fabs(uy) * adr + fabs(ux) * adc);
      }
      if (clamped) dS = aS = 0.0;
      if (gp) gp[p * G + g] = (double)scales[g] * dS;
      if (gp_abs) gp_abs[p * G + g] = fabs((double)scales[g]) * aS;
      if (gs) gs[g] += sig * dS;
      if (gs_abs) gs_abs[g] += fabs(sig) * aS;
    }
  }
  return 0;
}

/* ----------------------------------------------- DCNv3's softmax weights (R18)
 * The largest weight is found by comparisons, which a NaN never wins; the
 * NaN then reaches every weight of its row through the sum.  With M = +inf,
 * exp(+inf - inf) is NaN; a row of -inf has M = -inf and -inf - -inf = NaN. */
int dcn4o_softmax_weights(const dcn4o_shape* s, int dtype, const void* om, double* out) {
  int32_t Ho, Wo;
  if (dcn4o_check(s, &Ho, &Wo)) return -1;
  const int K = s->kh * s->kw;
  const int64_t rows = (int64_t)s->N * Ho * Wo * s->G;
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t base = r * 3 * K;
    for (int i = 0; i < 2 * K; ++i) out[base + i] = load_f32(dtype, om, base + i);
    double M = -INFINITY;
    for (int k = 0; k < K; ++k) {
      const double m = load_f32(dtype, om, base + 2 * K + k);
      if (m > M) M = m;
    }
    double sum = 0.0;
    for (int k = 0; k < K; ++k) sum += exp((double)load_f32(dtype, om, base + 2 * K + k) - M);
    for (int k = 0; k < K; ++k)
      out[base + 2 * K + k] = exp((double)load_f32(dtype, om, base + 2 * K + k) - M) / sum;
  }
  return 0;
}

/* ------------------------------------------------- merged offset/weight layer
 * The producer of the offset/weight tensor: one linear layer maps every
 * pixel's Cin features to its G*3K offsets and weights ([DCNv4 digest]
 * "方法3": offsets and weights from one merged linear layer), so
 *   om[r, j] = sum_k feat[r, k] * weight[j, k] + bias[j]
 * for rows r < M (pixels), outputs j < Nout; feat and weight in the I/O dtype,
 * bias fp32.  fp64 throughout; absum (nullable) receives
 * sum_k |feat*weight| + |bias| per output (tolerance bounds). */
int dcn4o_linear_f64(int64_t M, int32_t Cin, int32_t Nout, int dtype,
                     const void* feat, const void* weight, const float* bias,
                     double* out, double* absum) {
  if (M < 0 || Cin < 1 || Nout < 1) return -1;
  for (int64_t r = 0; r < M; ++r) {
    for (int32_t j = 0; j < Nout; ++j) {
      double acc = 0.0, a = 0.0;
      for (int32_t k = 0; k < Cin; ++k) {
        const double t = (double)load_f32(dtype, feat, r * Cin + k) *
                         (double)load_f32(dtype, weight, (int64_t)j * Cin + k);
        acc += t;
        a += fabs(t);
      }
      const double b = bias ? (double)bias[j] : 0.0;
      out[r * Nout + j] = acc + b;
      if (absum) absum[r * Nout + j] = a + fabs(b);
    }
  }
  return 0;
}

/* ------------------------------------------------ depthwise 3x3 convolution */

int dcn4o_dwconv3x3(int32_t N, int32_t H, int32_t W, int32_t C, int dtype,
                    const void* x, const void* w, const float* bias,
                    double* out64, void* out_raw) {
  if (N < 0 || H < 1 || W < 1 || C < 1) return -1;
  for (int64_t n = 0; n < N; ++n)
    for (int32_t y = 0; y < H; ++y)
      for (int32_t xx = 0; xx < W; ++xx)
        for (int32_t c = 0; c < C; ++c) {
          double s64 = 0.0;
          float acc = 0.0f;
          for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) {
              const int32_t yy = y + i - 1, xs = xx + j - 1;
              if (yy < 0 || yy >= H || xs < 0 || xs >= W) continue;  /* zero padding */
              const float wv = load_f32(dtype, w, (int64_t)(i * 3 + j) * C + c);
              const float xv = load_f32(dtype, x, ((n * H + yy) * W + xs) * (int64_t)C + c);
              s64 += (double)wv * (double)xv;
              acc = fmaf(wv, xv, acc);
            }
          const int64_t o = ((n * H + y) * W + xx) * (int64_t)C + c;
          if (bias) {
            s64 += (double)bias[c];
            acc = acc + bias[c];
          }
          if (out64) out64[o] = s64;
          if (out_raw) store_io(dtype, out_raw, o, acc);
        }
  return 0;
}
