// dcn4_api.cpp -- the C ABI of libdcn4.so: argument validation, planning and
// error reporting.  No HIP call is made before the arguments have passed
// validation, so every error path runs without a GPU.
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <new>

#include <hip/hip_runtime_api.h>

#include "dcn4.h"
#include "dcn4_internal.h"

namespace {

thread_local char g_last_error[256] = "";

dcn4_status fail(dcn4_status s, const char* msg) {
  snprintf(g_last_error, sizeof g_last_error, "%s", msg);
  return s;
}

bool aligned_to(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

constexpr int64_t kCoordLimit = int64_t(1) << 20;
// Margin of the tiled kernel's LDS window, in pixels around the footprint of
// the tile's undisplaced sample points: offsets within it gather from LDS.
constexpr int32_t kDefaultTileMargin = 4;
// In group-scale mode a group's points sit at s_g times the grid (FlowDCN's
// scale priors reach 4), so they spread further from the tile's footprint:
// one pixel more (measured with offset/weight rows read into registers:
// FlowDCN tokens 102.6 us at margin 4, 95.7 at 5, 97.4 at 6; the U-Net
// block, standard mode, 117.7 at 4, 121.0 at 5).
constexpr int32_t kDefaultTileMarginGroupScale = 5;
// lane-index bit (plus one) that swaps a lane's vector pairs in the tiled
// kernel: bit 3, so lanes 8 apart start on different LDS banks
constexpr int32_t kDefaultTileSwizzle = 4;

// Output size of the convolution index arithmetic with padding and dilation.
int64_t out_size(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d) {
  const int64_t span = in + 2 * p - d * (k - 1) - 1;
  return span < 0 ? 0 : span / s + 1;
}

dcn4_status validate_desc(const dcn4_desc& d, int64_t* Ho, int64_t* Wo) {
  if (d.dtype != DCN4_F32 && d.dtype != DCN4_BF16 && d.dtype != DCN4_F16)
    return fail(DCN4_ERR_INVALID_ARG, "dtype must be DCN4_F32, DCN4_BF16 or DCN4_F16");
  if (d.N < 0 || d.H < 1 || d.W < 1 || d.C < 1 || d.group < 1)
    return fail(DCN4_ERR_INVALID_ARG, "N must be >= 0 and H, W, C, group >= 1");
  if (d.C % d.group)
    return fail(DCN4_ERR_INVALID_ARG, "C must be a multiple of group");
  if (d.kernel_h < 1 || d.kernel_w < 1 || d.stride_h < 1 || d.stride_w < 1 ||
      d.dilation_h < 1 || d.dilation_w < 1 || d.pad_h < 0 || d.pad_w < 0)
    return fail(DCN4_ERR_INVALID_ARG,
                "kernel, stride and dilation must be >= 1 and pad >= 0");
  if (d.H > kCoordLimit || d.W > kCoordLimit || d.pad_h > kCoordLimit ||
      d.pad_w > kCoordLimit || d.stride_h > kCoordLimit || d.stride_w > kCoordLimit ||
      int64_t(d.dilation_h) * d.kernel_h > kCoordLimit ||
      int64_t(d.dilation_w) * d.kernel_w > kCoordLimit)
    return fail(DCN4_ERR_INVALID_ARG,
                "H, W, pads, strides and dilation*kernel must be <= 2^20");
  if (!isfinite(d.offset_scale))
    return fail(DCN4_ERR_INVALID_ARG, "offset_scale must be finite");
  if (d.use_group_scales) {
    if (!(d.kernel_h & 1) || !(d.kernel_w & 1))
      return fail(DCN4_ERR_INVALID_ARG, "group-scale mode needs odd kernel sizes");
    if (d.dilation_h != 1 || d.dilation_w != 1 || d.offset_scale != 1.0f)
      return fail(DCN4_ERR_INVALID_ARG,
                  "group-scale mode needs dilation 1 and offset_scale 1");
  }
  if (!(d.max_scale >= 0.0f))
    return fail(DCN4_ERR_INVALID_ARG, "max_scale must be 0 (none) or positive");
  if ((d.use_pixel_scales || d.max_scale > 0.0f) && !d.use_group_scales)
    return fail(DCN4_ERR_INVALID_ARG,
                "pixel scales and max_scale need group-scale mode");
  *Ho = out_size(d.H, d.kernel_h, d.stride_h, d.pad_h, d.dilation_h);
  *Wo = out_size(d.W, d.kernel_w, d.stride_w, d.pad_w, d.dilation_w);
  if (*Ho < 1 || *Wo < 1)
    return fail(DCN4_ERR_INVALID_ARG, "the output would be empty");
  return DCN4_OK;
}

// Channels per lane on the vector path: prefer 16 channels (fewer geometry
// instructions per channel) when the group allows it.
int32_t default_dp(int32_t D, int32_t es) {
  const int32_t vec = 16 / es;
  if ((D * es) % 16) return 0;
  const int32_t order_half[] = {2, 3, 1, 4};
  const int32_t order_f32[] = {4, 2, 3, 1};
  const int32_t* order = es == 4 ? order_f32 : order_half;
  for (int t = 0; t < 4; ++t)
    if (D % (order[t] * vec) == 0) return order[t] * vec;
  return 0;
}

}  // namespace

extern "C" {

dcn4_status dcn4_create(const dcn4_desc* desc, dcn4_plan** plan) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan output pointer is NULL");
  *plan = nullptr;
  if (!desc) return fail(DCN4_ERR_NULL, "descriptor is NULL");
  int64_t Ho = 0, Wo = 0;
  dcn4_status s = validate_desc(*desc, &Ho, &Wo);
  if (s != DCN4_OK) return s;

  dcn4::Plan p{};
  p.desc = *desc;
  p.Ho = (int32_t)Ho;
  p.Wo = (int32_t)Wo;
  p.D = desc->C / desc->group;
  p.K = desc->kernel_h * desc->kernel_w;
  p.es = desc->dtype == DCN4_F32 ? 4 : 2;
  p.mode = desc->use_group_scales ? dcn4::kGroupScale
           : desc->offset_scale == 1.0f ? dcn4::kStdUnitScale
                                        : dcn4::kStdScaled;
  p.dp_default = default_dp(p.D, p.es);
  p.dp = p.dp_default;
  p.kernel_choice = dcn4::kKernelAuto;
  p.tile_margin = desc->use_group_scales ? kDefaultTileMarginGroupScale : kDefaultTileMargin;
  p.tile_groups = 0;
  p.tile_pad = 0;
  p.tile_swizzle = kDefaultTileSwizzle;
  p.tile_window = 0;
  p.tile_passes = 0;
  p.tile_passes_x = 0;
  p.f16_window = 1;
  p.tile_om_unit = 0;
  dcn4::resolve_tile(p);

  // size limits of the 32-bit device arithmetic
  const int64_t pix = Ho * Wo;
  const int64_t x_img = int64_t(desc->H) * desc->W * desc->C * p.es;
  const int64_t lanes_img = pix * desc->C;  // worst case: one channel per lane
  const int64_t lim = (int64_t(1) << 31) - (int64_t(1) << 16);
  if (lanes_img >= lim || pix * desc->group * 3 * p.K * p.es >= lim ||
      pix * desc->C * p.es >= lim)
    return fail(DCN4_ERR_UNSUPPORTED, "one image's tensors exceed 2^31 bytes");
  // corner offsets use 24-bit multiplies: pixel index and pixel bytes
  if (int64_t(desc->H) * desc->W >= (int64_t(1) << 23) ||
      int64_t(desc->C) * p.es >= (int64_t(1) << 23))
    return fail(DCN4_ERR_UNSUPPORTED, "H*W and C*element bytes must be below 2^23");
  // a workgroup touches at most kBlock + 1 pixels; its gathers address the
  // images those pixels belong to from one 32-bit offset
  const int64_t span_images = (dcn4::kBlock + 1) / pix + 2;
  if (span_images * x_img >= lim)
    return fail(DCN4_ERR_UNSUPPORTED, "input images too large for 32-bit offsets");
  p.images_per_launch = (int32_t)(lim / (lanes_img > 0 ? lanes_img : 1));
  if (p.images_per_launch < 1) p.images_per_launch = 1;
  if (dcn4::forward_block(p, p.dp ? p.D / p.dp : p.D) == 0 ||
      dcn4::forward_block(p, p.D) == 0)
    return fail(DCN4_ERR_UNSUPPORTED,
                "offset/weight rows of one pixel are too large for LDS");

  const int64_t in_el = int64_t(desc->N) * desc->H * desc->W * desc->C;
  const int64_t out_el = int64_t(desc->N) * pix * desc->C;
  const int64_t om_el = int64_t(desc->N) * pix * desc->group * 3 * p.K;
  p.ideal_bytes = uint64_t(in_el + out_el + om_el) * p.es +
                  (desc->use_group_scales ? 4ull * desc->group : 0ull) +
                  (desc->use_pixel_scales ? 4ull * desc->N * pix * desc->group : 0ull);

  dcn4_plan* out = new (std::nothrow) dcn4_plan;
  if (!out) return fail(DCN4_ERR_NOMEM, "plan allocation failed");
  out->p = p;
  *plan = out;
  return DCN4_OK;
}

dcn4_status dcn4_query(const dcn4_plan* plan, int32_t* Ho, int32_t* Wo,
                       uint64_t* ideal_bytes) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  if (Ho) *Ho = plan->p.Ho;
  if (Wo) *Wo = plan->p.Wo;
  if (ideal_bytes) *ideal_bytes = plan->p.ideal_bytes;
  return DCN4_OK;
}

dcn4_status dcn4_plan_info(const dcn4_plan* plan, dcn4_launch_info* info) {
  if (!plan || !info) return fail(DCN4_ERR_NULL, "plan or info is NULL");
  const dcn4::Plan& p = plan->p;
  *info = dcn4_launch_info{};
  const bool vec = p.dp > 0;
  const int32_t dp = vec ? p.dp : 1;
  info->channels_per_lane = dp;
  info->vector_bytes = vec ? 16 : p.es;
  info->lanes_per_group = p.D / dp;
  const int32_t bwd_lds = (vec && p.kernel_choice != dcn4::kKernelDirect)
                              ? dcn4::tiled_backward_lds(p) : 0;
  info->backward_kernel = bwd_lds > 0 ? 2 : 1;
  info->backward_lds_bytes = bwd_lds;
  info->bucket_capacity = (int32_t)dcn4::bucket_capacity(p);
  if (vec && p.tile.ok) {
    const dcn4::TileShape& t = p.tile;
    info->channels_per_lane = t.dp;
    info->lanes_per_group = p.D / t.dp;
    const int64_t rows = t.th * (t.passes > 0 ? t.passes : 1);  // output rows per workgroup
    const int64_t cols = t.tw * (t.passes_x > 0 ? t.passes_x : 1);  // and columns
    const int64_t tiles = int64_t((p.Ho + rows - 1) / rows) * ((p.Wo + cols - 1) / cols);
    const int64_t per_image = tiles * (p.desc.group / t.gb) * t.slices;
    const int64_t imgs = (int64_t(1) << 30) / per_image;
    info->kernel = 2;
    info->block_threads = dcn4::kBlock;
    info->blocks = per_image * p.desc.N;
    info->launches = p.desc.N ? (int32_t)((p.desc.N + imgs - 1) / imgs) : 0;
    info->lds_bytes = t.fwd_lds_bytes;
    info->tile_h = t.th;
    info->tile_w = t.tw;
    info->tile_groups = t.gb;
    info->tile_margin = t.margin;
    info->tile_slices = t.slices;
    info->tile_window = t.whole ? 2 : 1;
    info->tile_passes = t.passes;
    info->tile_passes_x = t.passes_x;
    info->tile_f16_window = dcn4::tile_f16_window(p);
    info->tile_om_unit = t.om_direct ? 1 : t.omu;
    return DCN4_OK;
  }
  info->kernel = 1;
  info->block_threads = dcn4::forward_block(p, p.D / dp);
  int64_t blocks = 0;
  int32_t launches = 0;
  for (int32_t n0 = 0; n0 < p.desc.N; n0 += p.images_per_launch) {
    const int32_t nb = p.desc.N - n0 < p.images_per_launch ? p.desc.N - n0
                                                           : p.images_per_launch;
    blocks += (int64_t(nb) * p.Ho * p.Wo * p.desc.group * (p.D / dp) +
               info->block_threads - 1) / info->block_threads;
    ++launches;
  }
  info->blocks = blocks;
  info->launches = launches;
  info->lds_bytes = dcn4::forward_lds_bytes(p, p.D / dp, info->block_threads);
  return DCN4_OK;
}

dcn4_status dcn4_plan_set_option(dcn4_plan* plan, int32_t option, int32_t value) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  dcn4::Plan q = plan->p;  // applied only if the result is valid
  switch (option) {
    case DCN4_OPT_CHANNELS_PER_LANE: {
      if (value == 0) {
        q.dp = q.dp_default;
        q.dp_user = 0;
        break;
      }
      const int32_t vec = 16 / q.es;
      if (value < vec || value % vec || value / vec > 4 || q.D % value || (q.D * q.es) % 16)
        return fail(DCN4_ERR_INVALID_ARG,
                    "channels_per_lane must be 1-4 vectors of 16 bytes and divide D");
      if (dcn4::forward_block(q, q.D / value) == 0)
        return fail(DCN4_ERR_UNSUPPORTED, "offset/weight rows are too large for LDS");
      q.dp = value;
      q.dp_user = 1;
      break;
    }
    case DCN4_OPT_KERNEL:
      if (value < 0 || value > 2) return fail(DCN4_ERR_INVALID_ARG, "kernel must be 0, 1 or 2");
      q.kernel_choice = value;
      break;
    case DCN4_OPT_TILE_MARGIN:
      if (value < 0 || value > 16) return fail(DCN4_ERR_INVALID_ARG, "tile margin must be 0-16");
      q.tile_margin = value;
      break;
    case DCN4_OPT_TILE_GROUPS:
      if (value < 0 || (value > 0 && q.desc.group % value))
        return fail(DCN4_ERR_INVALID_ARG, "tile groups must divide G");
      q.tile_groups = value;
      break;
    case DCN4_OPT_TILE_PAD:
      if (value != 0 && value != 1) return fail(DCN4_ERR_INVALID_ARG, "tile pad must be 0 or 1");
      q.tile_pad = value;
      break;
    case DCN4_OPT_TILE_SWIZZLE:
      if (value < 0 || value > 6) return fail(DCN4_ERR_INVALID_ARG, "tile swizzle must be 0-6");
      q.tile_swizzle = value;
      break;
    case DCN4_OPT_TILE_WINDOW:
      if (value < 0 || value > 2) return fail(DCN4_ERR_INVALID_ARG, "tile window must be 0, 1 or 2");
      q.tile_window = value;
      break;
    case DCN4_OPT_TILE_PASSES:
      if (value < 0 || value > 64) return fail(DCN4_ERR_INVALID_ARG, "tile passes must be 0-64");
      q.tile_passes = value;
      break;
    case DCN4_OPT_TILE_PASSES_X:
      if (value < 0 || value > 64) return fail(DCN4_ERR_INVALID_ARG, "tile passes x must be 0-64");
      q.tile_passes_x = value;
      break;
    case DCN4_OPT_TILE_OM_UNIT:
      if (value != 0 && value != 1 && value != 4 && value != 16)
        return fail(DCN4_ERR_INVALID_ARG, "tile om unit must be 0, 1, 4 or 16");
      q.tile_om_unit = value;
      break;
    case DCN4_OPT_TILE_F16_WINDOW:
      if (value < 0 || value > 2)
        return fail(DCN4_ERR_INVALID_ARG, "tile f16 window must be 0, 1 or 2");
      q.f16_window = value;
      break;
    case DCN4_OPT_BUCKET_CAPACITY:
      if (value < 0 || value > 1024)
        return fail(DCN4_ERR_INVALID_ARG, "bucket capacity must be 0-1024");
      q.bucket_cap = value;
      break;
    default:
      return fail(DCN4_ERR_INVALID_ARG, "unknown option");
  }
  dcn4::resolve_tile(q);
  if (q.kernel_choice == dcn4::kKernelTiled && !q.tile.ok)
    return fail(DCN4_ERR_UNSUPPORTED, "the tiled kernel does not apply to this plan");
  plan->p = q;
  return DCN4_OK;
}

// Whether the byte ranges [a, a + na) and [b, b + nb) intersect (an empty or
// NULL range intersects nothing).
static bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Byte sizes of a plan's tensors.
struct IoBytes {
  uint64_t x, om, y, scales, pscales;
};
static IoBytes io_bytes(const dcn4::Plan& p) {
  const dcn4_desc& d = p.desc;
  const uint64_t pix = uint64_t(d.N) * p.Ho * p.Wo;
  IoBytes b;
  b.x = uint64_t(d.N) * d.H * d.W * d.C * p.es;
  b.om = pix * d.group * 3 * p.K * p.es;
  b.y = pix * d.C * p.es;
  b.scales = d.use_group_scales ? 4ull * d.group : 0;
  b.pscales = d.use_pixel_scales ? 4ull * pix * d.group : 0;
  return b;
}

// An output range that intersects any input range of the call.
static bool output_overlaps_inputs(const dcn4::Plan& p, const void* out, uint64_t n,
                                   const void* x, const void* om, const float* scales,
                                   const float* pscales, const void* gy) {
  const IoBytes b = io_bytes(p);
  return overlaps(out, n, x, b.x) || overlaps(out, n, om, b.om) ||
         overlaps(out, n, scales, b.scales) || overlaps(out, n, pscales, b.pscales) ||
         overlaps(out, n, gy, b.y);
}

static dcn4_status check_io(const dcn4::Plan& p, const void* x, const void* om,
                            const float* scales, const float* pscales,
                            const void* y, bool need_x) {
  if (!p.desc.use_pixel_scales && pscales)
    return fail(DCN4_ERR_INVALID_ARG,
                "pixel_scales given but the plan does not use pixel scales");
  if (p.desc.N == 0) return DCN4_OK;
  if (p.desc.use_pixel_scales && !pscales)
    return fail(DCN4_ERR_NULL, "pixel_scales is required by this plan");
  if (pscales && !aligned_to(pscales, 4))
    return fail(DCN4_ERR_MISALIGNED, "pixel_scales not 4-byte aligned");
  if ((need_x && (!x || !y)) || !om)
    return fail(DCN4_ERR_NULL, "x, offset_mask and y must not be NULL");
  if (p.desc.use_group_scales && !scales)
    return fail(DCN4_ERR_NULL, "group_scales is required in group-scale mode");
  if (!p.desc.use_group_scales && scales)
    return fail(DCN4_ERR_INVALID_ARG,
                "group_scales given but the plan is not in group-scale mode");
  const uintptr_t es = (uintptr_t)p.es;
  if ((need_x && (!aligned_to(x, es) || !aligned_to(y, es))) || !aligned_to(om, es))
    return fail(DCN4_ERR_MISALIGNED, "tensor pointer not aligned to its element size");
  if (scales && !aligned_to(scales, 4))
    return fail(DCN4_ERR_MISALIGNED, "group_scales not 4-byte aligned");
  return DCN4_OK;
}

dcn4_status dcn4_forward_scaled(const dcn4_plan* plan, const void* x,
                                const void* offset_mask,
                                const float* group_scales,
                                const float* pixel_scales, void* y,
                                void* stream) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  const dcn4::Plan& p = plan->p;
  dcn4_status s = check_io(p, x, offset_mask, group_scales, pixel_scales, y, true);
  if (s != DCN4_OK || p.desc.N == 0) return s;
  if (output_overlaps_inputs(p, y, io_bytes(p).y, x, offset_mask, group_scales, pixel_scales,
                             nullptr))
    return fail(DCN4_ERR_INVALID_ARG, "y overlaps an input");
  const bool vector_path = p.dp > 0 && aligned_to(x, 16) &&
                           aligned_to(offset_mask, 16) && aligned_to(y, 16);
  if (vector_path && p.tile.ok)
    s = dcn4::launch_tiled(p, x, offset_mask, group_scales, pixel_scales, y, stream);
  else
    s = dcn4::launch_forward(p, x, offset_mask, group_scales, pixel_scales, y,
                             stream, vector_path);
  if (s != DCN4_OK) return fail(s, dcn4::last_hip_error());
  return DCN4_OK;
}

dcn4_status dcn4_forward(const dcn4_plan* plan, const void* x,
                         const void* offset_mask, const float* group_scales,
                         void* y, void* stream) {
  if (plan && plan->p.desc.use_pixel_scales)
    return fail(DCN4_ERR_INVALID_ARG,
                "the plan takes pixel scales: call dcn4_forward_scaled");
  return dcn4_forward_scaled(plan, x, offset_mask, group_scales, nullptr, y, stream);
}

dcn4_status dcn4_dcnv3_softmax(const dcn4_plan* plan, const void* offset_mask, void* out,
                               void* stream) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  const dcn4::Plan& p = plan->p;
  if (p.desc.use_group_scales)
    return fail(DCN4_ERR_UNSUPPORTED, "the DCNv3-style path takes the standard geometry only");
  if (p.desc.N == 0) return DCN4_OK;
  if (!offset_mask || !out) return fail(DCN4_ERR_NULL, "offset_mask and out must not be NULL");
  if (!aligned_to(offset_mask, (uintptr_t)p.es) || !aligned_to(out, (uintptr_t)p.es))
    return fail(DCN4_ERR_MISALIGNED, "tensor pointer not aligned to its element size");
  const uint64_t n = io_bytes(p).om;
  if (overlaps(out, n, offset_mask, n)) return fail(DCN4_ERR_INVALID_ARG, "out overlaps offset_mask");
  const dcn4_status s = dcn4::launch_dcnv3_softmax(p, offset_mask, out, stream);
  if (s == DCN4_ERR_UNSUPPORTED)
    return fail(s, "offset/weight rows too large for the softmax pass");
  if (s != DCN4_OK) return fail(s, dcn4::last_hip_error());
  return DCN4_OK;
}

dcn4_status dcn4_dcnv3_forward(const dcn4_plan* plan, const void* x, const void* offset_mask,
                               void* y, void* stream) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  const dcn4::Plan& p = plan->p;
  if (p.desc.use_group_scales)
    return fail(DCN4_ERR_UNSUPPORTED, "the DCNv3-style path takes the standard geometry only");
  dcn4_status s = check_io(p, x, offset_mask, nullptr, nullptr, y, true);
  if (s != DCN4_OK || p.desc.N == 0) return s;
  if (output_overlaps_inputs(p, y, io_bytes(p).y, x, offset_mask, nullptr, nullptr, nullptr))
    return fail(DCN4_ERR_INVALID_ARG, "y overlaps an input");
  s = dcn4::launch_dcnv3(p, x, offset_mask, y, stream);
  if (s != DCN4_OK) return fail(s, dcn4::last_hip_error());
  return DCN4_OK;
}

dcn4_status dcn4_backward_workspace_size(const dcn4_plan* plan, uint64_t* bytes) {
  if (!plan || !bytes) return fail(DCN4_ERR_NULL, "plan or bytes is NULL");
  *bytes = dcn4::backward_workspace_bytes(plan->p);
  return DCN4_OK;
}

static dcn4_status check_backward(const dcn4::Plan& p, const void* x, const void* om,
                                  const float* scales, const float* pscales, const void* gy,
                                  const float* gx, const float* gom) {
  const dcn4_status s = check_io(p, x, om, scales, pscales, gy, true);
  if (s != DCN4_OK) return s;
  if ((gx && !aligned_to(gx, 4)) || (gom && !aligned_to(gom, 4)))
    return fail(DCN4_ERR_MISALIGNED, "gradient outputs must be 4-byte aligned");
  const IoBytes b = io_bytes(p);
  const uint64_t ngx = b.x / p.es * 4, ngom = b.om / p.es * 4;
  if (output_overlaps_inputs(p, gx, ngx, x, om, scales, pscales, gy) ||
      output_overlaps_inputs(p, gom, ngom, x, om, scales, pscales, gy) ||
      overlaps(gx, ngx, gom, ngom))
    return fail(DCN4_ERR_INVALID_ARG, "a gradient output overlaps an input or the other output");
  return DCN4_OK;
}

// The backward with a workspace of ws_bytes >= min_bytes (or none: atomic
// scatter); the chunks of the gathered grad_x are as large as fit ws_bytes.
static dcn4_status backward_with(const dcn4::Plan& p, const void* x, const void* offset_mask,
                                 const float* group_scales, const float* pixel_scales,
                                 const void* grad_y, float* grad_x, float* grad_offset_mask,
                                 void* workspace, uint64_t ws_bytes, uint64_t min_bytes,
                                 const char* too_small, void* stream) {
  dcn4_status s = check_backward(p, x, offset_mask, group_scales, pixel_scales, grad_y, grad_x,
                                 grad_offset_mask);
  if (s != DCN4_OK) return s;
  const uint64_t need = dcn4::backward_workspace_bytes(p);
  if (workspace && need) {
    if (!aligned_to(workspace, 256))
      return fail(DCN4_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    if (ws_bytes < min_bytes) return fail(DCN4_ERR_INVALID_ARG, too_small);
    const IoBytes b = io_bytes(p);
    if (output_overlaps_inputs(p, workspace, ws_bytes, x, offset_mask, group_scales,
                               pixel_scales, grad_y) ||
        overlaps(workspace, ws_bytes, grad_x, b.x / p.es * 4) ||
        overlaps(workspace, ws_bytes, grad_offset_mask, b.om / p.es * 4))
      return fail(DCN4_ERR_INVALID_ARG, "the workspace overlaps another argument");
  }
  if (p.desc.N == 0) return DCN4_OK;
  const bool vector_path = p.dp > 0 && aligned_to(x, 16) && aligned_to(offset_mask, 16) &&
                           aligned_to(grad_y, 16);
  s = dcn4::launch_backward(p, x, offset_mask, group_scales, pixel_scales, grad_y, grad_x,
                            grad_offset_mask, need ? workspace : nullptr,
                            need ? ws_bytes : 0, stream, vector_path);
  if (s != DCN4_OK) return fail(s, dcn4::last_hip_error());
  return DCN4_OK;
}

dcn4_status dcn4_backward_ws(const dcn4_plan* plan, const void* x, const void* offset_mask,
                             const float* group_scales, const float* pixel_scales,
                             const void* grad_y, float* grad_x, float* grad_offset_mask,
                             void* workspace, uint64_t workspace_bytes, void* stream) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  const dcn4::Plan& p = plan->p;
  return backward_with(p, x, offset_mask, group_scales, pixel_scales, grad_y, grad_x,
                       grad_offset_mask, workspace, workspace_bytes,
                       dcn4::backward_workspace_bytes(p),
                       "workspace smaller than dcn4_backward_workspace_size", stream);
}

dcn4_status dcn4_backward(const dcn4_plan* plan, const void* x,
                          const void* offset_mask, const float* group_scales,
                          const float* pixel_scales, const void* grad_y,
                          float* grad_x, float* grad_offset_mask, void* stream) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  const uint64_t need = dcn4::backward_workspace_bytes(plan->p);
  if (!grad_x || !need || plan->p.desc.N == 0)
    return dcn4_backward_ws(plan, x, offset_mask, group_scales, pixel_scales, grad_y, grad_x,
                            grad_offset_mask, nullptr, 0, stream);
  // validated before allocating, so a rejected call allocates nothing
  dcn4_status s = check_backward(plan->p, x, offset_mask, group_scales, pixel_scales, grad_y,
                                 grad_x, grad_offset_mask);
  if (s != DCN4_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (hipMallocAsync(&ws, need, st) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DCN4_ERR_HIP, "allocating the backward workspace failed");
  }
  s = dcn4_backward_ws(plan, x, offset_mask, group_scales, pixel_scales, grad_y, grad_x,
                       grad_offset_mask, ws, need, stream);
  if (hipFreeAsync(ws, st) != hipSuccess && s == DCN4_OK)
    return fail(DCN4_ERR_HIP, "freeing the backward workspace failed");
  return s;
}

dcn4_status dcn4_backward_scales(const dcn4_plan* plan, const void* x,
                                 const void* offset_mask, const float* group_scales,
                                 const float* pixel_scales, const void* grad_y,
                                 float* grad_group_scales, float* grad_pixel_scales,
                                 void* stream) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  const dcn4::Plan& p = plan->p;
  if (!p.desc.use_group_scales)
    return fail(DCN4_ERR_INVALID_ARG, "the plan has no group scales");
  if (grad_pixel_scales && !p.desc.use_pixel_scales)
    return fail(DCN4_ERR_INVALID_ARG, "grad_pixel_scales given but the plan has no pixel scales");
  if ((int64_t)p.desc.group * 4 > 64 * 1024)
    return fail(DCN4_ERR_UNSUPPORTED, "more than 16384 groups");
  dcn4_status s = check_io(p, x, offset_mask, group_scales, pixel_scales, grad_y, true);
  if (s != DCN4_OK) return s;
  if ((grad_group_scales && !aligned_to(grad_group_scales, 4)) ||
      (grad_pixel_scales && !aligned_to(grad_pixel_scales, 4)))
    return fail(DCN4_ERR_MISALIGNED, "gradient outputs must be 4-byte aligned");
  const IoBytes b = io_bytes(p);
  const uint64_t ngs = 4ull * p.desc.group;
  if (output_overlaps_inputs(p, grad_group_scales, ngs, x, offset_mask, group_scales,
                             pixel_scales, grad_y) ||
      output_overlaps_inputs(p, grad_pixel_scales, b.pscales, x, offset_mask, group_scales,
                             pixel_scales, grad_y) ||
      overlaps(grad_group_scales, ngs, grad_pixel_scales, b.pscales))
    return fail(DCN4_ERR_INVALID_ARG, "a gradient output overlaps an input or the other output");
  if (p.desc.N == 0) {
    if (!grad_group_scales) return DCN4_OK;  // the group gradient is still written: zeros
  } else if (!grad_group_scales && !grad_pixel_scales) {
    return DCN4_OK;
  }
  s = dcn4::launch_scale_grads(p, x, offset_mask, group_scales, pixel_scales, grad_y,
                               grad_group_scales, grad_pixel_scales, stream);
  if (s != DCN4_OK) return fail(s, dcn4::last_hip_error());
  return DCN4_OK;
}

dcn4_status dcn4_backward_noalloc(const dcn4_plan* plan, const void* x,
                                  const void* offset_mask, const float* group_scales,
                                  const float* pixel_scales, const void* grad_y,
                                  float* grad_x, float* grad_offset_mask, void* stream) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  const dcn4::Plan& p = plan->p;
  const uint64_t need = dcn4::backward_workspace_bytes(p);
  // only the gathered grad_x uses a workspace; without it this is dcn4_backward_ws
  if (!grad_x || !need || p.desc.N == 0)
    return dcn4_backward_ws(plan, x, offset_mask, group_scales, pixel_scales, grad_y, grad_x,
                            grad_offset_mask, nullptr, 0, stream);
  dcn4_status s = check_backward(p, x, offset_mask, group_scales, pixel_scales, grad_y, grad_x,
                                 grad_offset_mask);
  if (s != DCN4_OK) return s;
  // the scratch holds chunks of as many (image, group) pairs as fit it
  if (dcn4::backward_min_workspace_bytes(p) > dcn4::kScratchBytes)
    return fail(DCN4_ERR_UNSUPPORTED,
                "one image and group of the gathered grad_x need more workspace than the "
                "library's 64 MiB static scratch: call dcn4_backward_ws");
  void* ws = nullptr;
  s = dcn4::scratch_address(&ws);
  if (s != DCN4_OK) return fail(s, s == DCN4_ERR_HIP ? dcn4::last_hip_error()
                                                     : "device index beyond 63");
  return backward_with(p, x, offset_mask, group_scales, pixel_scales, grad_y, grad_x,
                       grad_offset_mask, ws, dcn4::kScratchBytes,
                       dcn4::backward_min_workspace_bytes(p), "static scratch too small", stream);
}

dcn4_status dcn4_offset_linear(const void* feat, const void* weight, const float* bias,
                               void* offset_mask, int64_t M, int32_t Cin, int32_t Nout,
                               int32_t dtype, void* stream) {
  if (dtype != DCN4_BF16 && dtype != DCN4_F16) {
    if (dtype == DCN4_F32)
      return fail(DCN4_ERR_UNSUPPORTED, "the offset/weight layer runs bf16 and fp16 only");
    return fail(DCN4_ERR_INVALID_ARG, "dtype must be DCN4_BF16 or DCN4_F16");
  }
  if (M < 0 || Cin < 1 || Nout < 1)
    return fail(DCN4_ERR_INVALID_ARG, "M must be >= 0 and Cin, Nout >= 1");
  if (Cin % 16)
    return fail(DCN4_ERR_UNSUPPORTED, "Cin must be a multiple of 16");
  // buffer offsets are 32-bit: the weight rows of every column chunk (up to
  // Nout rounded up to the chunk width) and one block of feature rows
  if ((int64_t(Nout) + dcn4::kLinearCols) * Cin * 2 > 0x7fffffff ||
      int64_t(dcn4::kLinearRows + 1) * Cin * 2 > 0x7fffffff)
    return fail(DCN4_ERR_UNSUPPORTED, "Cin * (Nout + 128) beyond 2^30 elements");
  if (M == 0) return DCN4_OK;
  if (!feat || !weight || !offset_mask)
    return fail(DCN4_ERR_NULL, "feat, weight and offset_mask must not be NULL");
  if (!aligned_to(feat, 16) || !aligned_to(weight, 16) || !aligned_to(offset_mask, 2) ||
      (bias && !aligned_to(bias, 4)))
    return fail(DCN4_ERR_MISALIGNED,
                "feat and weight must be 16-byte aligned, offset_mask 2, bias 4");
  const uint64_t nout = uint64_t(M) * Nout * 2;
  if (overlaps(offset_mask, nout, feat, uint64_t(M) * Cin * 2) ||
      overlaps(offset_mask, nout, weight, uint64_t(Nout) * Cin * 2) ||
      overlaps(offset_mask, nout, bias, bias ? 4ull * Nout : 0))
    return fail(DCN4_ERR_INVALID_ARG, "offset_mask overlaps feat, weight or bias");
  dcn4_status s = dcn4::launch_linear(feat, weight, bias, offset_mask, M, Cin, Nout, dtype,
                                      stream);
  if (s != DCN4_OK) return fail(s, dcn4::last_hip_error());
  return DCN4_OK;
}

dcn4_status dcn4_dwconv3x3(const void* x, const void* weight, const float* bias, void* out,
                           int32_t N, int32_t H, int32_t W, int32_t C, int32_t dtype,
                           void* stream) {
  if (dtype != DCN4_F32 && dtype != DCN4_BF16 && dtype != DCN4_F16)
    return fail(DCN4_ERR_INVALID_ARG, "dtype must be DCN4_F32, DCN4_BF16 or DCN4_F16");
  if (N < 0 || H < 1 || W < 1 || C < 1)
    return fail(DCN4_ERR_INVALID_ARG, "N must be >= 0 and H, W, C >= 1");
  if (N == 0) return DCN4_OK;
  if (!x || !weight || !out) return fail(DCN4_ERR_NULL, "x, weight and out must not be NULL");
  const uintptr_t es = dtype == DCN4_F32 ? 4 : 2;
  if (!aligned_to(x, es) || !aligned_to(weight, es) || !aligned_to(out, es) ||
      (bias && !aligned_to(bias, 4)))
    return fail(DCN4_ERR_MISALIGNED, "tensors must be aligned to the element size, bias to 4");
  const uint64_t nx = uint64_t(N) * H * W * C * es;
  if (overlaps(out, nx, x, nx) || overlaps(out, nx, weight, 9ull * C * es) ||
      overlaps(out, nx, bias, bias ? 4ull * C : 0))
    return fail(DCN4_ERR_INVALID_ARG, "out overlaps x, weight or bias");
  const bool vector_path = (C * es) % 16 == 0 && aligned_to(x, 16) && aligned_to(weight, 16) &&
                           aligned_to(out, 16) && (!bias || aligned_to(bias, 16));
  dcn4_status s = dcn4::launch_dwconv(x, weight, bias, out, N, H, W, C, dtype, vector_path,
                                      stream);
  if (s != DCN4_OK) return fail(s, s == DCN4_ERR_HIP ? dcn4::last_hip_error()
                                                     : "more than 2^31 workgroups");
  return DCN4_OK;
}

dcn4_status dcn4_probe_geometry(const dcn4_plan* plan, const void* offset_mask,
                                const float* group_scales,
                                const float* pixel_scales, int32_t* y0,
                                int32_t* x0, float* lh, float* lw,
                                uint8_t* inside, void* stream) {
  if (!plan) return fail(DCN4_ERR_NULL, "plan is NULL");
  const dcn4::Plan& p = plan->p;
  dcn4_status s = check_io(p, nullptr, offset_mask, group_scales, pixel_scales,
                           nullptr, false);
  if (s != DCN4_OK || p.desc.N == 0) return s;
  if (!y0 || !x0 || !lh || !lw || !inside)
    return fail(DCN4_ERR_NULL, "probe outputs must not be NULL");
  if (!aligned_to(y0, 4) || !aligned_to(x0, 4) || !aligned_to(lh, 4) || !aligned_to(lw, 4))
    return fail(DCN4_ERR_MISALIGNED, "probe outputs must be 4-byte aligned");
  s = dcn4::launch_probe(p, offset_mask, group_scales, pixel_scales, y0, x0, lh, lw,
                         inside, stream);
  if (s != DCN4_OK) return fail(s, dcn4::last_hip_error());
  return DCN4_OK;
}

void dcn4_destroy(dcn4_plan* plan) { delete plan; }

const char* dcn4_status_string(dcn4_status s) {
  switch (s) {
    case DCN4_OK: return "DCN4_OK";
    case DCN4_ERR_INVALID_ARG: return "DCN4_ERR_INVALID_ARG: invalid argument";
    case DCN4_ERR_UNSUPPORTED: return "DCN4_ERR_UNSUPPORTED: beyond size limits";
    case DCN4_ERR_MISALIGNED: return "DCN4_ERR_MISALIGNED: misaligned pointer";
    case DCN4_ERR_NULL: return "DCN4_ERR_NULL: required pointer is NULL";
    case DCN4_ERR_HIP: return "DCN4_ERR_HIP: HIP runtime error";
    case DCN4_ERR_NOMEM: return "DCN4_ERR_NOMEM: out of host memory";
  }
  return "unknown dcn4_status";
}

const char* dcn4_last_error(void) { return g_last_error; }

}  // extern "C"
