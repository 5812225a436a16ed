/*
 * dcn4_oracle.h -- CPU oracle for the DCNv4 forward spatial aggregation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under dynamic_sparse_vision_dcn4_amd/) shares no code, header,
 * table or helper with it, and neither side includes or links the other.
 *
 * Sources the oracle follows (web pages, cited by title and section):
 *   [DCNv4 digest]   CSDN, "（论文速读）DCNv4：高效可变形卷积算子"
 *                    - section 1 "移除Softmax归一化": aggregation weights are
 *                      unbounded, no softmax over the K points;
 *                    - section 2 "内存访问优化", "GPU效率的理论分析": bilinear
 *                      sampling (4 corners) at each of the 3x3 points, the
 *                      36HWC count and the 2HWC+27HWG ideal traffic model;
 *                    - "方法1. 消除冗余工作负载": the D=C/G channels of a group
 *                      share the sampling offsets and the weights;
 *                    - "方法2": channel-last layout;
 *                    - "方法3": offsets and weights come from one merged
 *                      linear layer (so they arrive in one tensor).
 *   [FlowDCN]        kler.cn, "NeurIPS'24 | FlowDCN：基于可变形卷积的任意分辨率
 *                    图像生成模型"
 *                    - section 2.2: sample location = pixel + kernel grid point
 *                      + predicted deformation, groups concatenated on channels;
 *                    - section 3.1: deformation split into a per-group scale
 *                      prior s_g and a predicted direction.
 *   [CANN Conv2D]    intelliparadigm, "CANN ops-nn 算子与 Stable Diffusion 的
 *                    卷积实现", section 2.1: the textbook convolution index
 *                    arithmetic (output y,x reads input y*s+i, x*s+j).
 *
 * Every reading taken where the pages are silent is listed next to the code
 * that takes it (grid origin, tap order, offset order, zero padding, the fp32
 * operation order, dtype of the offset/weight tensor).
 */
#ifndef DCN4_ORACLE_H
#define DCN4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { DCN4O_F32 = 0, DCN4O_BF16 = 1, DCN4O_F16 = 2 };

typedef struct {
  int32_t N, H, W, C, G;          /* input [N,H,W,C] channel-last, G groups   */
  int32_t kh, kw;                 /* kernel taps, K = kh*kw                    */
  int32_t sh, sw, ph, pw, dh, dw; /* stride, zero padding, dilation           */
  float offset_scale;             /* multiplies the predicted offset (std mode)*/
  int32_t multiscale;             /* 1: FlowDCN groupwise multi-scale geometry */
  int32_t pixel_scales;           /* 1: per-pixel scales [N,Ho,Wo,G] times s_g */
  float max_scale;                /* > 0: clamp of the effective scale (Smax)  */
} dcn4o_shape;

/* Validates the shape and returns the output size.  0 on success, -1 if the
 * shape is invalid (non-positive size, C % G != 0, empty output, a multi-scale
 * shape with an even kernel, dilation != 1 or offset_scale != 1, pixel scales
 * without multi-scale, a negative or NaN max_scale). */
int dcn4o_check(const dcn4o_shape* s, int32_t* Ho, int32_t* Wo);

/* Element codecs (exact decode; round-to-nearest-even encode). */
float dcn4o_bf16_to_f32(uint16_t h);
float dcn4o_f16_to_f32(uint16_t h);
uint16_t dcn4o_f32_to_bf16(float f);
uint16_t dcn4o_f32_to_f16(float f);

/* The definition, evaluated in fp64 (positions, weights, products, sum).
 * x: [N,H,W,C], om: [N,Ho,Wo,G,3K] in the I/O dtype `dtype`, scales: [G] fp32
 * (multi-scale only, else ignored), pscales: [N,Ho,Wo,G] fp32 (pixel_scales
 * only, else ignored).  y: fp64 output.
 * pix == NULL: all N*Ho*Wo output pixels, y is [N,Ho,Wo,C].
 * pix != NULL: only the npix listed flat pixel indices (n*Ho+yo)*Wo+xo, y is
 * [npix,C].  Returns 0 or -1 (invalid shape / pixel index). */
int dcn4o_forward_f64(const dcn4o_shape* s, int dtype, const void* x,
                      const void* om, const float* scales, const float* pscales,
                      double* y, const int64_t* pix, int64_t npix, int nthreads);

/* The same sum evaluated in fp32 with a fixed operation order (the reading of
 * "fp32 accumulation"), output rounded to the I/O dtype.  `acc` (nullable)
 * receives the fp32 accumulator before rounding. */
int dcn4o_forward_f32(const dcn4o_shape* s, int dtype, const void* x,
                      const void* om, const float* scales, const float* pscales,
                      void* y, float* acc, const int64_t* pix, int64_t npix,
                      int nthreads);

/* Sampling geometry of the fp32 evaluation, one entry per (pixel, g, k):
 * inside = the integer part of the location is in [-1,H-1]x[-1,W-1]; for
 * inside samples y0, x0 = integer parts, lh, lw = fractions (else all zero). */
int dcn4o_geometry(const dcn4o_shape* s, int dtype, const void* om,
                   const float* scales, const float* pscales, int32_t* y0,
                   int32_t* x0, float* lh, float* lw, uint8_t* inside,
                   const int64_t* pix, int64_t npix);

/* Counts gathered while running the fp64 definition over every output:
 * corner_terms = bilinear corner multiply-adds the definition contains
 * (4 per sample point per channel, padded corners included);
 * inbounds_terms = those whose corner lies inside the image. */
int dcn4o_count_terms(const dcn4o_shape* s, int dtype, const void* om,
                      const float* scales, const float* pscales,
                      int64_t* corner_terms, int64_t* inbounds_terms);

/* Gradients of the forward pass for an upstream gradient gy [N,Ho,Wo,C] in
 * the I/O dtype: gx [N,H,W,C] (dL/dx), gom [N,Ho,Wo,G,3K] (dL/d offsets and
 * dL/d weights, in the offset/weight layout), both fp64, either may be NULL.
 * The sampling decisions (cell, fractions, inside test, effective scale) are
 * the fp32 evaluation's; all arithmetic after them is fp64.  gx_abs/gom_abs
 * (nullable) receive the sums of the absolute values of every output's terms
 * and *max_terms the largest term count of any output (tolerance bounds). */
int dcn4o_backward(const dcn4o_shape* s, int dtype, const void* x,
                   const void* om, const float* scales, const float* pscales,
                   const void* gy, double* gx, double* gom, double* gx_abs,
                   double* gom_abs, int64_t* max_terms);

/* Gradients of the group scales (group-scale mode): gs [G] = dL/ds_g and,
 * for plans with pixel scales, gp [N,Ho,Wo,G] = dL/dsigma, both fp64 and
 * nullable, for an upstream gradient gy; the location moves by
 * u = fl(grid + direction) per unit of the effective scale, which is
 * s_g * sigma below the clamp and the constant Smax above it.  Sampling
 * decisions of the fp32 evaluation, fp64 arithmetic after them; gs_abs and
 * gp_abs (nullable) receive the sums of the absolute values of the terms.
 * 0, or -1 for a plan without group scales (or gp without pixel scales). */
int dcn4o_backward_scales(const dcn4o_shape* s, int dtype, const void* x,
                          const void* om, const float* scales, const float* pscales,
                          const void* gy, double* gs, double* gs_abs, double* gp,
                          double* gp_abs);

/* The merged linear layer that produces the offset/weight tensor
 * ([DCNv4 digest] "方法3"): out[r, j] = sum_k feat[r, k] * weight[j, k] +
 * bias[j], feat [M, Cin] and weight [Nout, Cin] in the I/O dtype, bias fp32
 * (nullable), out fp64 [M, Nout]; absum (nullable) receives the sum of the
 * absolute values of every output's terms.  0 or -1 (bad sizes). */
int dcn4o_linear_f64(int64_t M, int32_t Cin, int32_t Nout, int dtype,
                     const void* feat, const void* weight, const float* bias,
                     double* out, double* absum);

/* The depthwise 3x3 convolution in front of the offset/weight layer
 * ([DCNv4 digest] "方法3": DCNv3's offset subnetwork without its LayerNorm
 * and GELU, the separable structure of Xception; optional):
 *   out[n,y,x,c] = sum_{i,j<3} w[i,j,c] * x[n, y+i-1, x+j-1, c] + bias[c],
 * stride 1, zero padding 1, x and out [N,H,W,C] and w [3,3,C] in the I/O
 * dtype, bias fp32 [C] (nullable).  out64 (nullable): the sum in fp64;
 * out_raw (nullable): the fp32 evaluation -- acc = fma(w, x, acc) over the
 * nine taps in row-major order (taps outside the image skipped), then
 * acc + bias, rounded once to the I/O dtype (nearest even).  0 or -1. */
int dcn4o_dwconv3x3(int32_t N, int32_t H, int32_t W, int32_t C, int dtype,
                    const void* x, const void* w, const float* bias,
                    double* out64, void* out_raw);

/* DCNv3's normalisation of the aggregation weights, the step DCNv4 removes
 * ([DCNv4 digest] abstract and section 1 "移除Softmax归一化": DCNv3 passes
 * the weights through a softmax, bounding them to (0, 1)).  Reading R18: a
 * softmax over the K weights of each (output pixel, group) row,
 *   w_k = exp(m_k - M) / sum_j exp(m_j - M),  M = the largest m_j,
 * the offsets unchanged.  om is [N,Ho,Wo,G,3K] in the I/O dtype (R4); out
 * (fp64, same shape) receives the offsets as decoded and the exact weights.
 * A NaN or +inf weight makes its whole row's weights NaN, as does a row of
 * -inf.  0 or -1 (invalid shape). */
int dcn4o_softmax_weights(const dcn4o_shape* s, int dtype, const void* om, double* out);

/* Ideal traffic of one forward pass in bytes: input + output feature maps
 * plus the offset/weight tensor, each read or written once, plus 4G bytes of
 * fp32 scales in multi-scale mode and 4*N*Ho*Wo*G bytes of pixel scales
 * ([DCNv4 digest], "GPU效率的理论分析"). */
int64_t dcn4o_ideal_bytes(const dcn4o_shape* s, int dtype);

#ifdef __cplusplus
}
#endif
#endif
