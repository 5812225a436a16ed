/*
 * dcn4.h -- C ABI of the MI355X (gfx950) DCNv4 forward spatial-aggregation
 * library, libdcn4.so.
 *
 * The operation (pages cited by title and section):
 *   [DCNv4 digest] CSDN "（论文速读）DCNv4：高效可变形卷积算子"
 *   [FlowDCN]      kler.cn "NeurIPS'24 | FlowDCN：基于可变形卷积的任意分辨率
 *                  图像生成模型"
 *   [CANN Conv2D]  intelliparadigm "CANN ops-nn 算子与 Stable Diffusion 的卷积
 *                  实现"
 *   [SD U-Net tutorial] framerc.cn "从ConvNet到Diffusion：手把手把DCNv4塞进
 *                  Stable Diffusion的U-Net里试试效果"
 *
 * For every output pixel (n, yo, xo) and channel group g (G groups of
 * D = C/G channels), K = kernel_h*kernel_w points are sampled from the input
 * by bilinear interpolation with zero padding and summed with per-point
 * weights m that are not normalised (no softmax; [DCNv4 digest] section 1).
 * All D channels of a group share the offsets and the weights ([DCNv4 digest]
 * "方法1"); the groups' outputs are concatenated along channels ([FlowDCN]
 * 2.2).  Point k = i*kernel_w + j of group g samples
 *   standard mode:    row = yo*stride_h - pad_h + i*dilation_h
 *                           + offset_scale*dy_k,   (col likewise with dx_k)
 *   group-scale mode: row = yo*stride_h - pad_h + (kernel_h-1)/2
 *                           + S*((i - (kernel_h-1)/2) + dy_k)
 *                     (FlowDCN groupwise multi-scale, [FlowDCN] 3.1; odd
 *                     kernels, dilation 1, offset_scale 1), where the scale
 *                     S = s_g, or with pixel scales S = s_g*sigma[n,yo,xo,g]
 *                     (the predicted scale of [FlowDCN] 3.1), and with
 *                     max_scale > 0 the smaller of S and max_scale (the
 *                     maximum scale Smax of [FlowDCN] 3.3; a NaN S stays NaN)
 * and y = sum_k m_k * bilinear(x, row, col).  The base location is the
 * convolution index of [CANN Conv2D] 2.1 with padding and dilation; the
 * output size is Ho = (H + 2*pad_h - dilation_h*(kernel_h-1) - 1)/stride_h + 1
 * (Wo likewise).
 *
 * Arithmetic: fp32 throughout.  Per sample the location is an exact integer
 * part plus a fraction: t = fl(offset_scale*d) (group-scale mode:
 * fl(S*fl(grid + d)), measured from the integer centre, with
 * S = fl(s_g*sigma) before the clamp); f = floor(t);
 * lh = fl(t - f); y0 = base + f (exact); the sample is skipped unless
 * -1 <= y0 <= H-1 and -1 <= x0 <= W-1 (a NaN displacement fails the test);
 * hh = 1 - lh (same for x); corner weights hh*hw, hh*lw, lh*hw, lh*lw for
 * corners (y0,x0), (y0,x0+1), (y0+1,x0), (y0+1,x0+1); coefficient fl(m*w);
 * corners outside the image are skipped; acc = fma(coefficient, value, acc)
 * with points outer and corners inner, starting from +0; the result is
 * rounded to the I/O dtype to nearest even.  Subnormals are kept.  Every
 * kernel variant and option gives bit-identical results.
 *
 * Layouts (all dense, channel-last, row-major):
 *   x            [N, H, W, C]          I/O dtype
 *   offset_mask  [N, Ho, Wo, G, 3K]    I/O dtype; per group the K interleaved
 *                                      (dx_k, dy_k) pairs (x along W), then
 *                                      the K weights m_k.  This is the single
 *                                      tensor a merged offset/weight linear
 *                                      layer emits ([DCNv4 digest] "方法3").
 *   group_scales [G]                   fp32, group-scale mode only
 *   pixel_scales [N, Ho, Wo, G]        fp32, plans with use_pixel_scales only
 *   y            [N, Ho, Wo, C]        I/O dtype
 *
 * Ownership and execution: the caller owns every buffer and the stream.  All
 * data pointers are device pointers.  No call allocates device memory except
 * dcn4_backward, which takes its workspace with hipMallocAsync on the call's
 * stream and returns it with hipFreeAsync (dcn4_backward_ws takes a
 * caller-owned workspace instead); a plan holds host-side metadata only and
 * is immutable after creation, so one plan may be used from several host
 * threads and streams at once.  Calls are asynchronous on `stream` (a
 * hipStream_t, NULL = the default stream) and never synchronise; buffers must
 * stay alive until the stream's work has completed.  No output may overlap
 * an input or another output of the same call: the byte ranges the plan
 * implies are compared before launching (DCN4_ERR_INVALID_ARG).
 *
 * Errors: every call returns a status and never throws across the ABI.
 * Arguments are validated before anything is launched, so an error status
 * means nothing was enqueued (except DCN4_ERR_HIP, reported by the runtime at
 * launch).  dcn4_last_error() gives a message for the calling thread's last
 * failed call.
 */
#ifndef DCN4_H
#define DCN4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DCN4_F32 = 0,  /* IEEE binary32 */
  DCN4_BF16 = 1, /* bfloat16 (upper half of a binary32) */
  DCN4_F16 = 2   /* IEEE binary16 */
} dcn4_dtype;

typedef enum {
  DCN4_OK = 0,
  DCN4_ERR_INVALID_ARG = -1, /* descriptor or argument not a valid operation */
  DCN4_ERR_UNSUPPORTED = -2, /* valid, but beyond this library's size limits */
  DCN4_ERR_MISALIGNED = -3,  /* pointer not aligned to its element size      */
  DCN4_ERR_NULL = -4,        /* required pointer is NULL                       */
  DCN4_ERR_HIP = -5,         /* the HIP runtime reported an error at launch    */
  DCN4_ERR_NOMEM = -6        /* host allocation of the plan failed             */
} dcn4_status;

/* Operation descriptor.  Valid when: N >= 0; H, W, C, group >= 1;
 * C % group == 0; kernel, stride, dilation >= 1; pad >= 0; the output size is
 * at least 1x1; H, W, pads, strides and dilation*kernel <= 2^20; offset_scale
 * finite.  With use_group_scales != 0 the kernel sizes must be odd and
 * dilation and offset_scale must be 1.  use_pixel_scales and a non-zero
 * max_scale need use_group_scales; max_scale must be 0 (no clamp) or a
 * positive number (+inf allowed). */
typedef struct {
  int32_t N, H, W, C, group;
  int32_t kernel_h, kernel_w;
  int32_t stride_h, stride_w;
  int32_t pad_h, pad_w;
  int32_t dilation_h, dilation_w;
  float offset_scale;       /* multiplies (dx, dy) in standard mode        */
  int32_t use_group_scales; /* 1: FlowDCN groupwise multi-scale geometry   */
  int32_t dtype;            /* dcn4_dtype of x, offset_mask and y          */
  int32_t use_pixel_scales; /* 1: per-pixel predicted scales times s_g     */
  float max_scale;          /* > 0: clamp of the effective scale; 0: none  */
} dcn4_desc;

typedef struct dcn4_plan dcn4_plan; /* opaque, immutable after creation */

/* Validates `desc`, chooses the kernel variant and launch shape, and returns
 * a plan in *plan (NULL on error).  The descriptor carries the module
 * arguments of the DCNv4 layer ([SD U-Net tutorial] 2.2: channels, kernel
 * size, stride, pad, dilation, group) with the output size of the
 * convolution index arithmetic ([CANN Conv2D] 2.1), plus FlowDCN's scale
 * options ([FlowDCN] 3.1, 3.3).  The plan is owned by the caller until
 * dcn4_destroy.  Errors: DCN4_ERR_NULL (desc or plan NULL),
 * DCN4_ERR_INVALID_ARG, DCN4_ERR_UNSUPPORTED (a single image's tensors beyond
 * 2^31 bytes), DCN4_ERR_NOMEM.  Makes no HIP call. */
dcn4_status dcn4_create(const dcn4_desc* desc, dcn4_plan** plan);

/* Output size and the ideal traffic of one forward pass in bytes: input and
 * output once, the offset/weight tensor once, plus 4G bytes of scales in
 * group-scale mode and 4*N*Ho*Wo*G bytes of pixel scales when the plan uses
 * them (the 2HWC + 27HWG element model of [DCNv4 digest]
 * "GPU效率的理论分析", with input and output at their own sizes).  Any output
 * pointer may be NULL.  Errors: DCN4_ERR_NULL (plan NULL). */
dcn4_status dcn4_query(const dcn4_plan* plan, int32_t* Ho, int32_t* Wo,
                       uint64_t* ideal_bytes);

/* Launch shape the plan chose (for tests, tuning and reports). */
typedef struct {
  int32_t kernel;            /* 1: direct gather kernel, 2: tiled kernel    */
  int32_t channels_per_lane; /* D' -- channels one lane owns                */
  int32_t vector_bytes;      /* bytes per load/store instruction (16 or es) */
  int32_t lanes_per_group;   /* D / D'                                      */
  int32_t block_threads;     /* threads per workgroup                       */
  int64_t blocks;            /* workgroups over all launches                */
  int32_t launches;          /* kernel launches per forward call            */
  int32_t lds_bytes;         /* dynamic LDS per workgroup                   */
  int32_t tile_h, tile_w;    /* tiled kernel: output tile                   */
  int32_t tile_groups;       /* tiled kernel: groups per workgroup          */
  int32_t tile_margin;       /* tiled kernel: window margin in pixels       */
  int32_t backward_kernel;   /* grad_offset_mask of dcn4_backward: 2 tiled
                                (LDS window) for 16-byte aligned tensors
                                when grad_x is gathered or not asked for;
                                1 direct otherwise: one lane per 16-byte
                                channel vector when the tensors allow it,
                                channel-strided lanes when they do not or
                                when grad_x is scattered (no workspace)     */
  int32_t backward_lds_bytes; /* dynamic LDS per tiled-backward workgroup   */
  int32_t tile_slices;       /* tiled kernel: channel slices per group (1:
                                a workgroup's window holds whole groups;
                                > 1: one slice of channels_per_lane
                                channels of one group, one lane per pixel) */
  int32_t bucket_capacity;   /* gathered grad_x: records per bucket          */
  int32_t tile_window;       /* tiled kernel's LDS window: 1 the tile's
                                footprint plus the margin, 2 the whole image
                                plus a one-pixel zero border (0: no tile)   */
  int32_t tile_passes;       /* tiled forward: tile rows a workgroup takes
                                under one staging of its window             */
  int32_t tile_f16_window;   /* tiled bf16 forward: a workgroup re-encodes
                                its window as fp16 whenever every value of
                                it converts exactly (the fma then widens the
                                value; other windows stay bf16): 1 through
                                registers while staging, 2 in LDS after the
                                copies; 0 never                             */
  int32_t tile_om_unit;      /* tiled forward: bytes per lane of an
                                offset/weight copy instruction (4 or 16),
                                or 1: rows read into registers, not staged */
  int32_t tile_passes_x;     /* tiled forward, whole-image window: tile
                                columns a workgroup takes under one staging
                                (1 otherwise)                               */
} dcn4_launch_info;

/* Fills *info for the plan as it would run with 16-byte aligned pointers.
 * Errors: DCN4_ERR_NULL. */
dcn4_status dcn4_plan_info(const dcn4_plan* plan, dcn4_launch_info* info);

/* Tuning options of a plan.  Every valid setting computes the identical
 * result; they change only how the work is mapped to the GPU. */
typedef enum {
  /* D': channels one lane owns, 1-4 vectors of 16 bytes dividing D; 0 = default */
  DCN4_OPT_CHANNELS_PER_LANE = 0,
  /* 0 = automatic, 1 = direct gather kernel, 2 = tiled kernel (LDS window) */
  DCN4_OPT_KERNEL = 1,
  /* tiled kernel: pixels of margin around the tile's footprint, 0-16;
   * default 4, 5 in group-scale mode */
  DCN4_OPT_TILE_MARGIN = 2,
  /* tiled kernel: groups per workgroup (a divisor of G); 0 = automatic */
  DCN4_OPT_TILE_GROUPS = 3,
  /* tiled kernel: 1 = pad each LDS window pixel to an odd number of 16-byte
   * chunks (fewer bank conflicts), 0 = no padding */
  DCN4_OPT_TILE_PAD = 4,
  /* tiled kernel: k = 1-6 makes lanes whose index has bit k-1 set read their
   * 16-byte vectors pairwise swapped (fewer LDS bank conflicts); 0 = off */
  DCN4_OPT_TILE_SWIZZLE = 5,
  /* backward, gathered grad_x: records per (cell, group) bucket, 1-1024;
   * samples beyond it are added by the overflow kernel's atomics; 0 =
   * automatic (the mean bucket load plus three Poisson standard deviations
   * plus 4, to a multiple of 4).  Changes the workspace size. */
  DCN4_OPT_BUCKET_CAPACITY = 6,
  /* tiled kernels' LDS window: 1 = the tile's footprint plus the margin (a
   * wave with a point whose corners leave it gathers that point from global
   * memory), 2 = the whole image plus a one-pixel zero border (no point
   * leaves it; only where it fits LDS), 0 = automatic (the whole image when
   * it fits and stages at most 1.25 times the bytes of the margin window) */
  DCN4_OPT_TILE_WINDOW = 7,
  /* tiled forward: tile rows each workgroup computes from one staging of
   * its window, 1-64 (at most the output's tile rows; fewer when the joint
   * window does not fit LDS).  Whole-image window: 0 = automatic (as many as
   * keep four workgroups per CU).  Margin window: the window covers the
   * rows' joint footprint plus the margin; 0 = one row. */
  DCN4_OPT_TILE_PASSES = 8,
  /* tiled bf16 forward: a workgroup whose window values are all zero or of
   * magnitude in [2^-17, 65280] (exactly representable in fp16) stages them
   * as fp16, which its fp32 fmas widen for free; other windows stay bf16.
   * 1 = re-encoded through registers while staging when the window takes
   * at most 10 staging passes (larger windows stay bf16); 2 = re-encoded in
   * LDS after the copies land, any window size; 0 = always bf16.  Default 1. */
  DCN4_OPT_TILE_F16_WINDOW = 9,
  /* tiled kernels: how a workgroup's offset/weight rows reach its lanes.
   * 4 or 16: staged in LDS by copy instructions of that many bytes per lane
   * (16: a quarter of the instructions, up to 14 padding bytes per pixel).
   * 1: the forward's lanes read their own rows from global memory into
   * registers, nothing staged (3x3 kernels with 16-bit values and one group
   * per workgroup; other plans, and the backward, stage 4-byte units).
   * 0 = automatic: 1 where it applies, else 16 when it keeps the
   * workgroups per compute unit, else 4.  Same results. */
  DCN4_OPT_TILE_OM_UNIT = 10,
  /* tiled forward under the whole-image window: tile columns each
   * workgroup computes from one staging of the image (with the rows of
   * DCN4_OPT_TILE_PASSES), 1-64, at most the output's tile columns;
   * 0 = automatic (one column).  No effect on the margin window. */
  DCN4_OPT_TILE_PASSES_X = 11
} dcn4_option;

/* Sets one option (see dcn4_option).  Errors: DCN4_ERR_NULL,
 * DCN4_ERR_INVALID_ARG (unknown option or value out of range),
 * DCN4_ERR_UNSUPPORTED (the tiled kernel was requested but does not apply to
 * this plan: groups that are not 16-byte multiples, offset/weight rows not
 * 4-byte aligned, or a window too large for LDS).  Not safe while another
 * thread uses the plan. */
dcn4_status dcn4_plan_set_option(dcn4_plan* plan, int32_t option, int32_t value);

/* Enqueues the forward pass y = DCNv4(x, offset_mask[, group_scales]) on
 * `stream`: the spatial aggregation defined at the top of this file ([DCNv4
 * digest] section 1 and "方法1"; [FlowDCN] 3.1 in group-scale mode), on the
 * channel-last layouts of [DCNv4 digest] "方法2".  x and offset_mask are read,
 * y [N, Ho, Wo, C] is written and must not overlap them (DCN4_ERR_INVALID_ARG).
 * group_scales must be non-NULL exactly when the plan uses group
 * scales.  Pointers must be aligned to the element size (4 B for fp32 and the
 * scales, 2 B otherwise); when x, offset_mask and y are 16-byte aligned and
 * D*es is a multiple of 16 the vectorised kernel runs, otherwise an
 * element-wise kernel computes the identical result.  N == 0 enqueues
 * nothing.  Errors: DCN4_ERR_NULL, DCN4_ERR_MISALIGNED, DCN4_ERR_INVALID_ARG
 * (scales given or missing against the plan's mode, or a plan that takes
 * pixel scales: those run through dcn4_forward_scaled), DCN4_ERR_HIP. */
dcn4_status dcn4_forward(const dcn4_plan* plan, const void* x,
                         const void* offset_mask, const float* group_scales,
                         void* y, void* stream);

/* The forward pass of a plan with FlowDCN's predicted per-pixel scales
 * ([FlowDCN] 3.1: the deformation split into a predicted scale and a
 * predicted direction; 3.3: the maximum scale Smax): pixel_scales is a device
 * array [N, Ho, Wo, G] of fp32, 4-byte aligned, required exactly when the
 * plan has use_pixel_scales (with NULL this is dcn4_forward).  Otherwise as
 * dcn4_forward. */
dcn4_status dcn4_forward_scaled(const dcn4_plan* plan, const void* x,
                                const void* offset_mask,
                                const float* group_scales,
                                const float* pixel_scales, void* y,
                                void* stream);

/* DCNv3-style comparison ([DCNv4 digest] abstract: DCNv4's forward pass is
 * reported more than three times as fast as DCNv3's; section 1: DCNv3
 * normalises the aggregation weights with a softmax; "方法1": DCNv3's kernel
 * gives each channel of each output position its own thread, which reads the
 * group's offsets and weights again).  Two calls, for plans in the standard
 * geometry (group-scale plans: DCN4_ERR_UNSUPPORTED):
 *
 * dcn4_dcnv3_softmax writes `out` = offset_mask with each (pixel, group)
 * row's K weights m_k replaced by exp(m_k - M) / sum_j exp(m_j - M), M the
 * row's largest weight, computed in fp32 (expf, the sum in point order, one
 * division) and rounded to the I/O dtype to nearest even; the offsets are
 * copied unchanged.  A NaN or +inf weight, or a row of -inf, makes the row's
 * weights NaN.  offset_mask and out are [N, Ho, Wo, G, 3K] in the I/O dtype,
 * aligned to the element size, and must not overlap (DCN4_ERR_INVALID_ARG).
 *
 * dcn4_dcnv3_forward computes exactly what dcn4_forward computes (the same
 * fp32 operations, bit for bit) with DCNv3's thread layout: one thread per
 * (output pixel, channel), each reading its group's offset/weight row from
 * global memory and computing the sampling geometry itself; pass it the
 * output of dcn4_dcnv3_softmax for DCNv3's operator.  Same arguments and
 * errors as dcn4_forward without scales.
 *
 * N == 0 enqueues nothing.  Errors: DCN4_ERR_NULL, DCN4_ERR_MISALIGNED,
 * DCN4_ERR_INVALID_ARG, DCN4_ERR_UNSUPPORTED, DCN4_ERR_HIP. */
dcn4_status dcn4_dcnv3_softmax(const dcn4_plan* plan, const void* offset_mask, void* out,
                               void* stream);
dcn4_status dcn4_dcnv3_forward(const dcn4_plan* plan, const void* x, const void* offset_mask,
                               void* y, void* stream);

/* Backward pass: the gradients of a loss L with respect to the input and to
 * the offset/weight tensor, given dL/dy.  grad_y is [N, Ho, Wo, C] in the I/O
 * dtype; grad_x [N, H, W, C] and grad_offset_mask [N, Ho, Wo, G, 3K] are fp32
 * device arrays, 4-byte aligned, either of them NULL to skip it; both are
 * overwritten.  In the offset/weight layout, grad_offset_mask holds
 * dL/d(dx_k, dy_k) and dL/dm_k:
 *   dL/dm_k  = sum over the group's channels c of dL/dy_c * B_c(p_k),
 *   dL/d(dy_k) = m_k * f * sum_c dL/dy_c * dB_c/drow, dL/d(dx_k) likewise
 *              with dB/dcol, f = offset_scale or the group's scale S,
 *   dL/dx[corner] = sum over the samples that read it of m_k * w * dL/dy,
 * where, in the cell (y0, x0) with fractions (lh, lw), dB/drow =
 * (1-lw)(v10-v00) + lw(v11-v01) and dB/dcol = (1-lh)(v01-v00) + lh(v11-v10):
 * the derivative from above at integer locations.  The sampling decisions
 * are the forward's (same device functions); a sample that is not inside has
 * zero gradient.  The gradients of the group and pixel scales come from
 * dcn4_backward_scales.
 * grad_x is the adjoint of the bilinear gather ([DCNv4 digest] "GPU效率的
 * 理论分析": every sample reads four corners of its group's D channels):
 * with a workspace each sample is appended to the bucket of its cell and
 * group and every input pixel gathers the buckets of the four cells it is a
 * corner of, accumulating fl(m_k*w) * dL/dy with fp32 fused multiply-adds;
 * without one every product fl(fl(m_k*w) * dL/dy) is added with an fp32
 * atomic.  Either way the order of the sum varies from run to run, so grad_x
 * is not bit-reproducible; the fp32 sums of grad_offset_mask are.  This entry point
 * allocates the workspace (dcn4_backward_workspace_size bytes) with
 * hipMallocAsync on `stream` and frees it with hipFreeAsync after the
 * launches; an allocation failure is DCN4_ERR_HIP.  Other arguments,
 * validation and errors as dcn4_forward_scaled (grad_y in the role of y). */
dcn4_status dcn4_backward(const dcn4_plan* plan, const void* x,
                          const void* offset_mask, const float* group_scales,
                          const float* pixel_scales, const void* grad_y,
                          float* grad_x, float* grad_offset_mask, void* stream);

/* Bytes of device workspace dcn4_backward_ws needs to gather grad_x.  The
 * gather runs over the batch in chunks of images x groups: at most as many
 * (image, group) pairs per chunk as fit the operator's ideal traffic bytes
 * (dcn4_query; at least one pair, at most 2 GiB), as few chunks as that
 * allows, of even size; a chunk's workspace is a
 * 256-byte counter, a 4-byte count per bucket ((H+1)*(W+1) cells per image
 * and group), a 4-byte overflow entry per sample (Ho*Wo*K per image and
 * group), each of these three rounded up to 256 bytes, and 16 * capacity
 * bytes of records per bucket.  0 when one image has 2^31 or more samples or
 * buckets: then grad_x is always scattered with atomics.  Errors:
 * DCN4_ERR_NULL. */
dcn4_status dcn4_backward_workspace_size(const dcn4_plan* plan, uint64_t* bytes);

/* dcn4_backward with a caller-owned workspace: `workspace` is a device
 * buffer of workspace_bytes bytes, 256-byte aligned (DCN4_ERR_MISALIGNED),
 * at least dcn4_backward_workspace_size (DCN4_ERR_INVALID_ARG), overlapping
 * no other argument; its contents on entry do not matter and on return are
 * undefined.  workspace NULL (or a size query of 0) selects the atomic
 * scatter for grad_x, which needs no workspace.  Calls that share a
 * workspace must be ordered (same stream, or synchronised). */
dcn4_status dcn4_backward_ws(const dcn4_plan* plan, const void* x,
                             const void* offset_mask, const float* group_scales,
                             const float* pixel_scales, const void* grad_y,
                             float* grad_x, float* grad_offset_mask,
                             void* workspace, uint64_t workspace_bytes,
                             void* stream);

/* Gradients of FlowDCN's scales ([FlowDCN] 3.1: the deformation's scale is
 * predicted per pixel by a linear layer of its own, on top of the group
 * prior; 3.3: the maximum scale), for plans in group-scale mode.  Point k
 * of group g samples centre + S * u_k on each axis, u_k = fl(grid_k + d_k),
 * so dL/dS = sum_k m_k (u_y,k sum_c dL/dy_c dB_c/drow + u_x,k sum_c dL/dy_c
 * dB_c/dcol) over the inside samples (the forward's sampling decisions, the
 * derivatives of dcn4_backward); below the clamp S = s_g * sigma, so
 *   grad_pixel_scales[n,yo,xo,g] = s_g * dL/dS   (plans with pixel scales)
 *   grad_group_scales[g]         = sum over pixels of sigma * dL/dS
 * (sigma = 1 without pixel scales); where fl(s_g * sigma) > max_scale the
 * scale is the constant max_scale and both are 0.  grad_group_scales [G] and
 * grad_pixel_scales [N, Ho, Wo, G] are fp32 device arrays, 4-byte aligned,
 * either NULL to skip it, both overwritten; the group sums are fp32 atomics
 * in no fixed order.  x, offset_mask, group_scales, pixel_scales and grad_y as
 * in dcn4_backward.  Errors: DCN4_ERR_INVALID_ARG (a plan without group
 * scales, grad_pixel_scales without pixel scales, an output overlapping an
 * input or the other output), DCN4_ERR_UNSUPPORTED (more than 16384 groups),
 * and those of dcn4_backward. */
dcn4_status dcn4_backward_scales(const dcn4_plan* plan, const void* x,
                                 const void* offset_mask, const float* group_scales,
                                 const float* pixel_scales, const void* grad_y,
                                 float* grad_group_scales, float* grad_pixel_scales,
                                 void* stream);

/* dcn4_backward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the gathered grad_x takes its workspace from a static device array of the
 * library, 64 MiB per GPU, held from the library's load until the process
 * ends, in chunks of as many (image, group) pairs as fit it; the call
 * allocates nothing.  A problem whose single (image, group) pair needs more
 * than 64 MiB is refused with DCN4_ERR_UNSUPPORTED before anything is
 * enqueued (use dcn4_backward_ws).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams, or threads without ordering) race and give
 * wrong gradients; calls ordered on one stream are safe.  The array's
 * counters are cleared by a kernel at the start of each call.  Arguments,
 * results, validation and other errors as dcn4_backward. */
dcn4_status dcn4_backward_noalloc(const dcn4_plan* plan, const void* x,
                                  const void* offset_mask, const float* group_scales,
                                  const float* pixel_scales, const void* grad_y,
                                  float* grad_x, float* grad_offset_mask, void* stream);

/* The producer of the offset/weight tensor: the merged linear layer of
 * [DCNv4 digest] "方法3" (offsets and weights from one linear layer),
 *   offset_mask[r, j] = sum_k feat[r, k] * weight[j, k] + bias[j],
 * r < M, j < Nout.  With M = N*Ho*Wo pixels and Nout = G*3K this writes the
 * offset_mask that dcn4_forward reads (the layer's output order is the
 * per-pixel [G, 3K] layout).  feat [M, Cin] and weight [Nout, Cin] row-major
 * in `dtype` (DCN4_BF16 or DCN4_F16; DCN4_F32 is DCN4_ERR_UNSUPPORTED), bias
 * fp32 [Nout] or NULL; products accumulated in fp32 on the matrix cores, the
 * sum plus bias rounded to `dtype` to nearest even.  Cin must be a multiple
 * of 16 (DCN4_ERR_UNSUPPORTED); feat and weight 16-byte aligned, offset_mask
 * 2-byte, bias 4-byte (DCN4_ERR_MISALIGNED); offset_mask must not overlap
 * feat, weight or bias (DCN4_ERR_INVALID_ARG).  M == 0 enqueues nothing.
 * Asynchronous on `stream`; the caller owns every buffer. */
dcn4_status dcn4_offset_linear(const void* feat, const void* weight,
                               const float* bias, void* offset_mask, int64_t M,
                               int32_t Cin, int32_t Nout, int32_t dtype,
                               void* stream);

/* The optional stage in front of the offset/weight layer: a depthwise 3x3
 * convolution ([DCNv4 digest] "方法3": DCNv3's offset subnetwork without its
 * LayerNorm and GELU, the separable structure of Xception; dropping it is
 * allowed when latency matters more),
 *   out[n,y,x,c] = sum_{i,j<3} weight[i,j,c] * x[n, y+i-1, x+j-1, c] + bias[c],
 * stride 1, zero padding 1.  x and out [N,H,W,C] and weight [3,3,C] (i along
 * H, j along W; a PyTorch depthwise weight [C,1,3,3] permuted to (2,3,0)) in
 * `dtype`, bias fp32 [C] or NULL.  fp32 arithmetic in a fixed order: an fma
 * per tap in row-major order, taps outside the image contributing nothing,
 * then the bias, one rounding to `dtype` (nearest even); the result does not
 * depend on the launch shape.  Pointers aligned to the element size (bias to
 * 4 bytes; DCN4_ERR_MISALIGNED); out must not overlap x, weight or bias
 * (DCN4_ERR_INVALID_ARG).
 * N == 0 enqueues nothing.  Asynchronous on `stream`; the caller owns every
 * buffer. */
dcn4_status dcn4_dwconv3x3(const void* x, const void* weight, const float* bias,
                           void* out, int32_t N, int32_t H, int32_t W, int32_t C,
                           int32_t dtype, void* stream);

/* Test probe of the sampling geometry: for every (n, yo, xo, g, k), in that
 * order, writes inside (1 if the integer parts passed the -1 <= y0 <= H-1,
 * -1 <= x0 <= W-1 test), and for inside samples the integer parts y0, x0 and
 * the fractions lh, lw of the arithmetic above (zeros otherwise), computed
 * by the same device functions as the forward kernels.  Outputs are device
 * arrays of N*Ho*Wo*G*K entries; pixel_scales as in dcn4_forward_scaled.
 * Errors as dcn4_forward_scaled. */
dcn4_status dcn4_probe_geometry(const dcn4_plan* plan, const void* offset_mask,
                                const float* group_scales,
                                const float* pixel_scales, int32_t* y0,
                                int32_t* x0, float* lh, float* lw,
                                uint8_t* inside, void* stream);

/* Frees a plan made by dcn4_create (the host-side description of one DCNv4
 * layer, [SD U-Net tutorial] 2.2); NULL is allowed.  The caller must not
 * destroy a plan while another thread is calling with it; work already
 * enqueued does not use the plan. */
void dcn4_destroy(dcn4_plan* plan);

/* Static description of a status code. */
const char* dcn4_status_string(dcn4_status status);

/* Message describing the calling thread's last failed call ("" if none). */
const char* dcn4_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
