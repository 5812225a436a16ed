// dcn4_kernels.hip -- DCNv4 forward spatial aggregation for CDNA4 (gfx950).
//
// Pages cited by title and section:
//   [DCNv4 digest] CSDN "（论文速读）DCNv4：高效可变形卷积算子"
//   [FlowDCN]      kler.cn "NeurIPS'24 | FlowDCN：基于可变形卷积的任意分辨率
//                  图像生成模型"
//
// Work decomposition.  A "lane item" is (output pixel, group g, channel slice
// l): the lane owns D' = VEC*NV contiguous channels of group g and computes
// the sample geometry and the bilinear coefficients once for all of them
// ([DCNv4 digest] "方法1": one thread per several channels of a group, so the
// offsets, weights and coefficients are read and computed once per D'
// channels).  Items are numbered pixel-major, group, slice, and a 256-thread
// workgroup takes 256 consecutive items.
//
// Memory.  The input and output are channel-last, so a lane's D' channels are
// contiguous and move with 128-bit loads and stores ([DCNv4 digest] "方法2").
// The offset/weight rows of the pixels a workgroup touches form one contiguous
// byte range of the merged tensor; the workgroup copies it to LDS with 128-bit
// loads and every lane reads its 3K values from there.  Corner gathers use
// raw buffer loads: an out-of-range offset returns zero, so a corner outside
// the image is fetched as 0 from a sentinel offset (no branch, no fault) and
// its coefficient is set to 0.  Accumulation is fp32 in registers.
//
// Placement.  MI355X dispatches consecutive workgroup ids round-robin over
// its 8 XCDs, each with its own L2.  Workgroup ids are remapped so that XCD x
// runs one contiguous range of items, i.e. a band of image rows, whose
// neighbouring gathers then hit that XCD's L2.
//
// Arithmetic order (every operation one IEEE fp32 op; built with
// -ffp-contract=off): location = base + fl(os*d) (group-scale mode: centre +
// fl(s_g*fl(grid + d))); inside iff -1<row<H and -1<col<W; y0 = floor(row),
// lh = row - y0, hh = 1 - lh; corner weights hh*hw, hh*lw, lh*hw, lh*lw;
// coefficient fl(m*w); acc = fma(coefficient, value, acc), points outer,
// corners (y0,x0), (y0,x0+1), (y0+1,x0), (y0+1,x0+1) inner; acc starts at +0.
// A corner outside the image adds fma(0, 0, acc) == acc exactly (acc is never
// -0 because it starts at +0), so the result equals skipping that corner.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "dcn4_internal.h"

namespace dcn4 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Word 3 of a gfx9 raw buffer descriptor: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;
// Offset that no descriptor covers: loads from it return zero.
constexpr uint32_t kOutside = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, kRsrcWord3);
}

// Global -> LDS copy without a register round trip: lane i of the wave writes
// its `bytes` (16 or 4) at lds_wave + i*bytes, so a wave fills one contiguous
// run; every load of a copy loop is in flight at once.  An out-of-range
// offset writes zeros.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void copy16_to_lds(rsrc_t r, char* lds_wave, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave, 16, (int)off, 0, 0, 0);
}
// The same with `unit` (4 or 16, wave-uniform) bytes per lane.
__device__ __forceinline__ void copy_unit_to_lds(int unit, rsrc_t r, char* lds_wave, uint32_t off) {
  if (unit == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave, 16, (int)off, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave, 4, (int)off, 0, 0, 0);
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// ------------------------------------------------------------ element codecs
template <int DT> struct Io;
template <> struct Io<DCN4_F32> {
  static constexpr int es = 4;
  typedef float raw;
  __device__ static float dec(raw r) { return r; }
  __device__ static float lane(u32x4 v, int e) { return __uint_as_float(v[e]); }
  __device__ static raw enc(float f) { return f; }
};
template <> struct Io<DCN4_BF16> {
  static constexpr int es = 2;
  typedef uint16_t raw;
  __device__ static float dec(raw r) { return __uint_as_float((uint32_t)r << 16); }
  __device__ static float lane(u32x4 v, int e) {
    uint32_t w = v[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  __device__ static raw enc(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);  // round to nearest even
  }
  // two values, packed low then high (one packed round-to-nearest-even convert)
  __device__ static uint32_t enc2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, b2));
  }
};
template <> struct Io<DCN4_F16> {
  static constexpr int es = 2;
  typedef uint16_t raw;
  __device__ static float dec(raw r) { return (float)__builtin_bit_cast(_Float16, r); }
  __device__ static float lane(u32x4 v, int e) {
    uint32_t w = v[e >> 1];
    return dec((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  __device__ static raw enc(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
  }
  __device__ static uint32_t enc2(float lo, float hi) {
    return (uint32_t)enc(lo) | ((uint32_t)enc(hi) << 16);
  }
};

// ------------------------------------------------------------ sample geometry
// Shared by the forward kernel and the geometry probe, so the probe reports
// exactly the locations the forward pass samples.  A location is an exact
// integer base plus a displacement t; the integer part is base + floor(t) and
// the fraction t - floor(t), so the fraction's accuracy does not depend on
// how far the pixel is from the origin.
struct Loc {
  float by, bx;  // exact integer base (standard) or centre (group-scale)
  float ty, tx;  // displacement from the base
};

// gy/gx: grid offset of the point from the centre (group-scale mode).
template <int MODE>
__device__ __forceinline__ Loc sample_location(float by, float bx, float gy,
                                               float gx, float dy, float dx,
                                               float os, float sg) {
  Loc l;
  l.by = by;
  l.bx = bx;
  if (MODE == kStdUnitScale) {
    l.ty = dy;
    l.tx = dx;
  } else if (MODE == kStdScaled) {
    l.ty = os * dy;
    l.tx = os * dx;
  } else {
    // [FlowDCN] 3.1: per-group scale prior times (grid point + direction)
    l.ty = sg * (gy + dy);
    l.tx = sg * (gx + dx);
  }
  return l;
}

struct Cell {
  int y0, x0;
  float yf, xf;  // integer parts as exact floats (compared before converting)
  float lh, lw;
  bool inside;
};

// inside: the integer part lies in [-1,H-1] x [-1,W-1] (NaN fails).  For an
// outside location y0/x0 are meaningless; every use of them is selected away
// by `inside` (selects never read the unused arm).
__device__ __forceinline__ Cell locate(Loc l, float Hm1, float Wm1) {
  Cell c;
  const float fy = __builtin_floorf(l.ty), fx = __builtin_floorf(l.tx);
  const float yf = l.by + fy, xf = l.bx + fx;  // exact while inside
  c.inside = (yf >= -1.0f) && (yf <= Hm1) && (xf >= -1.0f) && (xf <= Wm1);
  c.yf = yf;
  c.xf = xf;
  c.y0 = (int)yf;
  c.x0 = (int)xf;
  c.lh = l.ty - fy;
  c.lw = l.tx - fx;
  return c;
}

// Group-scale mode: the scale of group g at output pixel p (counted from the
// launch's first image): the group prior s_g, times the predicted scale of
// ([FlowDCN] 3.1) when the plan has pixel scales, replaced by the maximum
// scale ([FlowDCN] 3.3) when larger; the comparison is false for NaN, so a NaN
// scale stays NaN and its samples land nowhere.
__device__ __forceinline__ float group_scale(const FwdArgs& a, uint64_t p, uint32_t g) {
  float S = a.scales[g];
  if (a.pscales) S = S * a.pscales[p * (uint32_t)a.G + g];
  if (a.max_scale > 0.0f && S > a.max_scale) S = a.max_scale;
  return S;
}

// XCD-aware workgroup order: hardware id b runs on XCD b % 8; XCD x gets the
// contiguous logical range [start_x, start_x + count_x).
__device__ __forceinline__ int xcd_block(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
}

// ------------------------------------------------------------ forward kernel
// Per-lane constants of the forward pass.
struct LaneCtx {
  int by0, bx0;        // base row/col of point (0,0) (centre in group-scale mode)
  int hy, hx;          // (k-1)/2 per axis, group-scale mode
  float sg;            // group scale (group-scale mode)
  uint32_t lane_bytes; // byte offset of the lane's channels in its image
  uint32_t pix_bytes, row_stride;
};

// Coefficients and corner offsets of one sample point (corners 00,01,10,11).
struct Tap {
  float c[4];
  uint32_t q[4];
};

// Point k's geometry from its decoded offsets and weight.
template <int MODE, int KS>
__device__ __forceinline__ Tap tap_geometry_v(const FwdArgs& a, const LaneCtx& t, float dx,
                                              float dy, float m, int k) {
  const int kw = KS ? KS : a.kw;
  const int i = k / kw, j = k - (k / kw) * kw;
  float by, bx, gy = 0.0f, gx = 0.0f;
  if (MODE == kGroupScale) {
    by = (float)t.by0;
    bx = (float)t.bx0;
    gy = (float)(i - t.hy);
    gx = (float)(j - t.hx);
  } else {
    by = (float)(t.by0 + i * a.dh);
    bx = (float)(t.bx0 + j * a.dw);
  }
  const Cell c = locate(sample_location<MODE>(by, bx, gy, gx, dy, dx,
                                              a.offset_scale, t.sg),
                        a.Hm1, a.Wm1);
  const bool vy0 = c.inside && c.y0 >= 0, vy1 = c.inside && c.y0 < a.H - 1;
  const bool vx0 = c.inside && c.x0 >= 0, vx1 = c.inside && c.x0 < a.W - 1;
  const float hh = 1.0f - c.lh, hw = 1.0f - c.lw;
  Tap r;
  r.c[0] = (vy0 && vx0) ? m * (hh * hw) : 0.0f;
  r.c[1] = (vy0 && vx1) ? m * (hh * c.lw) : 0.0f;
  r.c[2] = (vy1 && vx0) ? m * (c.lh * hw) : 0.0f;
  r.c[3] = (vy1 && vx1) ? m * (c.lh * c.lw) : 0.0f;
  // pixel index within the lane's image fits 24 signed bits (H*W < 2^23)
  const uint32_t o00 = t.lane_bytes +
      (uint32_t)__mul24(__mul24(c.y0, a.W) + c.x0, (int)t.pix_bytes);
  r.q[0] = (vy0 && vx0) ? o00 : kOutside;
  r.q[1] = (vy0 && vx1) ? o00 + t.pix_bytes : kOutside;
  r.q[2] = (vy1 && vx0) ? o00 + t.row_stride : kOutside;
  r.q[3] = (vy1 && vx1) ? o00 + t.row_stride + t.pix_bytes : kOutside;
  return r;
}

// The same with point k's values read from the pixel's offset/weight row.
template <int DT, int MODE, int KS>
__device__ __forceinline__ Tap tap_geometry(const FwdArgs& a, const LaneCtx& t,
                                            const typename Io<DT>::raw* om, int k) {
  typedef Io<DT> io;
  const int K = KS ? KS * KS : a.kh * a.kw;
  return tap_geometry_v<MODE, KS>(a, t, io::dec(om[2 * k]), io::dec(om[2 * k + 1]),
                                  io::dec(om[2 * K + k]), k);
}

// The four corners' values of one point: NV 16-byte vectors per corner, or
// (element path) DP single elements widened to fp32.
template <int DT, int VEC, int NV> struct TapData {
  u32x4 v[4][NV];
  __device__ __forceinline__ void load(rsrc_t xr, const Tap& g) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int n = 0; n < NV; ++n)
        v[q][n] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(g.q[q] + 16 * n), 0, 0);
  }
  // The same with the vectors of each pair swapped when r16 == 16: slot n
  // holds vector n ^ 1 (the tiled kernel's per-lane vector order).  Offsets
  // stay non-negative: slot 2j at q + 16r + 32j, slot 2j+1 at q + 16(1-r) + 32j.
  __device__ __forceinline__ void load_swapped(rsrc_t xr, const Tap& g, uint32_t r16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t qe = g.q[q] + r16, qo = g.q[q] + (16u - r16);
#pragma unroll
      for (int n = 0; n < NV; ++n)
        v[q][n] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, (int)(((n & 1) ? qo : qe) + 16 * (n & ~1)), 0, 0);
    }
  }
  __device__ __forceinline__ void accumulate(float* acc, const Tap& g) const {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          acc[n * VEC + e] = __builtin_fmaf(g.c[q], Io<DT>::lane(v[q][n], e), acc[n * VEC + e]);
  }
};
template <int DT, int NV> struct TapData<DT, 1, NV> {
  float v[4][NV];
  __device__ __forceinline__ void load(rsrc_t xr, const Tap& g) {
    typedef Io<DT> io;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        if (io::es == 4)
          v[q][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, (int)(g.q[q] + 4 * e), 0, 0));
        else
          v[q][e] = io::dec((typename io::raw)__builtin_amdgcn_raw_buffer_load_b16(xr, (int)(g.q[q] + 2 * e), 0, 0));
      }
  }
  __device__ __forceinline__ void accumulate(float* acc, const Tap& g) const {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < NV; ++e) acc[e] = __builtin_fmaf(g.c[q], v[q][e], acc[e]);
  }
};

// DT: I/O dtype; VEC: elements per load (16/es, or 1 on the element path);
// NV: loads per corner (D' = VEC*NV); MODE: geometry; KS: 3 for a 3x3
// kernel known at compile time, 0 for run-time kernel sizes.
// Register budget: up to 128 VGPRs (4 waves per SIMD) for D' <= 2 vectors,
// more for the wider lanes whose two point buffers need them.
template <int DT, int VEC, int NV, int MODE, int KS>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(NV <= 2 ? 4 : (NV == 3 ? 3 : 2))))
void dcn4_forward_kernel(FwdArgs a) {
  typedef Io<DT> io;
  constexpr int es = io::es;
  constexpr int DP = VEC * NV;
  extern __shared__ u32x4 lds_rows[];

  const int lb = xcd_block(blockIdx.x, a.nblocks);
  const int item0 = lb * a.block;
  const int item_last = min(item0 + a.block, a.total_items) - 1;

  // ---- stage the offset/weight rows of the pixels this workgroup touches
  const uint32_t p_first = fastdiv((uint32_t)item0, a.div_ipp);
  const uint32_t p_last = fastdiv((uint32_t)item_last, a.div_ipp);
  // The copy starts at the 16-byte boundary at or below the first row (an
  // absolute address, so a tensor that is only element-aligned still gets
  // aligned vector loads; the lead bytes lie in the same 16-byte chunk as
  // the first row).  Bytes past the last row are not fetched (range check).
  const uint64_t row_bytes = (uint64_t)a.rowel * es;
  const char* first_row = a.om + (uint64_t)p_first * row_bytes;
  const uint32_t lead = (uint32_t)((uintptr_t)first_row & 15u);
  const char* aligned = first_row - lead;
  const uint32_t len = lead + (uint32_t)((uint64_t)(p_last + 1 - p_first) * row_bytes);
  {
    const rsrc_t r = make_rsrc(aligned, (len + 3u) & ~3u);
    const uint32_t nvec = (len + 15u) >> 4;
    const uint32_t lane = threadIdx.x & 63u;
    for (uint32_t base = threadIdx.x & ~63u; base < nvec; base += (uint32_t)a.block) {
      const uint32_t v = base + lane;
      if (v < nvec)
        copy16_to_lds(r, reinterpret_cast<char*>(lds_rows) + base * 16u, v << 4);
    }
  }
  __syncthreads();

  const int item = item0 + (int)threadIdx.x;
  if (item >= a.total_items) return;

  // ---- which pixel, group and channel slice this lane owns
  const uint32_t p = fastdiv((uint32_t)item, a.div_ipp);
  const uint32_t r_in_pix = (uint32_t)item - p * (uint32_t)a.ipp;
  const uint32_t g = fastdiv(r_in_pix, a.div_L);
  const uint32_t l = r_in_pix - g * (uint32_t)a.L;
  const uint32_t n = fastdiv(p, a.div_hw);
  const uint32_t rem = p - n * (uint32_t)(a.Ho * a.Wo);
  const uint32_t yo = fastdiv(rem, a.div_wo);
  const uint32_t xo = rem - yo * (uint32_t)a.Wo;
  const int K = KS ? KS * KS : a.kh * a.kw;

  // offset/weight row of (p, g) in LDS, as raw elements
  const typename io::raw* om =
      reinterpret_cast<const typename io::raw*>(lds_rows) + lead / es +
      (p - p_first) * (uint32_t)a.rowel + g * (uint32_t)(3 * K);

  // input: buffer based at the first image this workgroup touches
  const uint32_t n_first = fastdiv(p_first, a.div_hw);
  const uint64_t x_base = (uint64_t)n_first * a.img_bytes;
  const uint64_t x_left = a.x_bytes - x_base;
  const rsrc_t xr = make_rsrc(a.x + x_base,
                              (uint32_t)(x_left < 0x7fffffffu ? x_left : 0x7fffffffu));
  LaneCtx t;
  t.pix_bytes = (uint32_t)a.C * es;
  t.row_stride = (uint32_t)a.W * t.pix_bytes;
  t.lane_bytes = (n - n_first) * a.img_bytes + (g * (uint32_t)a.D + l * DP) * es;
  t.sg = (MODE == kGroupScale) ? group_scale(a, p, g) : 1.0f;
  t.hy = ((KS ? KS : a.kh) - 1) >> 1;
  t.hx = ((KS ? KS : a.kw) - 1) >> 1;
  t.by0 = (int)yo * a.sh - a.ph + (MODE == kGroupScale ? t.hy : 0);
  t.bx0 = (int)xo * a.sw - a.pw + (MODE == kGroupScale ? t.hx : 0);

  float acc[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) acc[e] = 0.0f;

  // ---- software pipeline over the K points, two buffers: the geometry and
  // the corner loads of the next point are issued before the multiply-adds
  // of the current one, so one point's gathers are in flight while the other
  // is accumulated.  The point index is wave-uniform (scalar registers); the
  // loop is not unrolled so the compiler cannot sink the multiply-adds of all
  // points below all the loads.
  Tap ga = tap_geometry<DT, MODE, KS>(a, t, om, 0), gb;
  TapData<DT, VEC, NV> da, db;
  da.load(xr, ga);
  int k = 0;
#pragma unroll 1
  for (; k + 1 < K; k += 2) {
    gb = tap_geometry<DT, MODE, KS>(a, t, om, k + 1);
    db.load(xr, gb);
    da.accumulate(acc, ga);
    if (k + 2 < K) {
      ga = tap_geometry<DT, MODE, KS>(a, t, om, k + 2);
      da.load(xr, ga);
    }
    db.accumulate(acc, gb);
  }
  if (k < K) da.accumulate(acc, ga);

  // ---- epilogue: round to the I/O dtype, store D' contiguous channels.
  // The empty asm pins each fp32 sum in a register, so the conversion is its
  // own rounding (the compiler would otherwise fuse the last fma with the
  // fp16 conversion into one rounding).
#pragma unroll
  for (int e = 0; e < DP; ++e) asm volatile("" : "+v"(acc[e]));
  char* yp = a.y + ((uint64_t)p * (uint32_t)a.C + g * (uint32_t)a.D + l * DP) * es;
  if (VEC > 1) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      u32x4 w;
      if (es == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(acc[v * VEC + e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)io::enc(acc[v * VEC + 2 * e]) |
                 ((uint32_t)io::enc(acc[v * VEC + 2 * e + 1]) << 16);
      }
      *reinterpret_cast<u32x4*>(yp + 16 * v) = w;
    }
  } else {
    typedef typename io::raw R;
#pragma unroll
    for (int e = 0; e < DP; ++e) reinterpret_cast<R*>(yp)[e] = io::enc(acc[e]);
  }
}


// ------------------------------------------------ DCNv3-style comparison
// DCNv3, the predecessor ([DCNv4 digest] abstract, section 1 and "方法1"),
// normalises each (pixel, group) row's K weights with a softmax, and its
// kernel gives every (output pixel, channel) a thread of its own, so the D
// threads of a group each read the group's offsets and weights from memory
// and each compute the same sampling geometry.  Built to measure DCNv4's
// design against on this GPU.  The arithmetic per output is R8's, so on the
// same offset/weight tensor the aggregation equals dcn4_forward bit for bit.

// Softmax pass: a workgroup owns R consecutive rows of the offset/weight
// tensor (R * 3K contiguous elements): coalesced element copies into LDS,
// one thread per row normalises its K weights in fp32 (the largest weight
// subtracted, expf, the sum in point order, one division, rounded to the
// I/O dtype), coalesced copies back out with the offsets unchanged.  The
// largest weight is found by comparisons a NaN never wins, so a NaN weight
// reaches the row's every weight through the sum.
template <int DT>
__global__ __launch_bounds__(kBlock) void dcn4_dcnv3_softmax_kernel(
    const typename Io<DT>::raw* in, typename Io<DT>::raw* out, uint64_t rows,
    int32_t K, int32_t R) {
  typedef Io<DT> io;
  typedef typename io::raw Rw;
  extern __shared__ u32x4 lds_softmax[];
  Rw* buf = reinterpret_cast<Rw*>(lds_softmax);
  const uint64_t row0 = (uint64_t)blockIdx.x * (uint32_t)R;
  const uint64_t left = rows - row0;
  const uint32_t nr = left < (uint64_t)R ? (uint32_t)left : (uint32_t)R;
  const uint32_t rowel = 3u * (uint32_t)K;
  const uint32_t nel = nr * rowel;
  const Rw* src = in + row0 * rowel;
  Rw* dst = out + row0 * rowel;
  for (uint32_t i = threadIdx.x; i < nel; i += kBlock) buf[i] = src[i];
  __syncthreads();
  if (threadIdx.x < nr) {
    Rw* w = buf + threadIdx.x * rowel + 2 * K;
    float M = -__builtin_inff();
    for (int k = 0; k < K; ++k) {
      const float m = io::dec(w[k]);
      if (m > M) M = m;
    }
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum += expf(io::dec(w[k]) - M);
    for (int k = 0; k < K; ++k) w[k] = io::enc(expf(io::dec(w[k]) - M) / sum);
  }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < nel; i += kBlock) dst[i] = buf[i];
}

// Aggregation: one thread per (output pixel, channel) of the launch, the
// channel fastest (a wave covers 64 consecutive channels of a pixel); the
// offset/weight row is read from global memory by each of its D threads;
// per point the direct kernel's geometry and one element per corner.
template <int DT, int MODE, int KS>
__global__ __launch_bounds__(kBlock) void dcn4_dcnv3_kernel(FwdArgs a) {
  typedef Io<DT> io;
  constexpr int es = io::es;
  const uint32_t item0 = blockIdx.x * (uint32_t)kBlock;
  const uint32_t item = item0 + threadIdx.x;
  if (item >= (uint32_t)a.total_items) return;
  const uint32_t p = fastdiv(item, a.div_ipp);  // ipp = C
  const uint32_t c = item - p * (uint32_t)a.C;
  const uint32_t g = fastdiv(c, a.div_L);       // L = D
  const uint32_t n = fastdiv(p, a.div_hw);
  const uint32_t rem = p - n * (uint32_t)(a.Ho * a.Wo);
  const uint32_t yo = fastdiv(rem, a.div_wo);
  const uint32_t xo = rem - yo * (uint32_t)a.Wo;
  const int K = KS ? KS * KS : a.kh * a.kw;
  const typename io::raw* om = reinterpret_cast<const typename io::raw*>(a.om) +
                               ((uint64_t)p * (uint32_t)a.G + g) * (uint32_t)(3 * K);

  // input buffer based at the image of the workgroup's first thread
  const uint32_t n_first = fastdiv(fastdiv(item0, a.div_ipp), a.div_hw);
  const uint64_t x_base = (uint64_t)n_first * a.img_bytes;
  const uint64_t x_left = a.x_bytes - x_base;
  const rsrc_t xr = make_rsrc(a.x + x_base,
                              (uint32_t)(x_left < 0x7fffffffu ? x_left : 0x7fffffffu));
  LaneCtx t;
  t.pix_bytes = (uint32_t)a.C * es;
  t.row_stride = (uint32_t)a.W * t.pix_bytes;
  t.lane_bytes = (n - n_first) * a.img_bytes + c * es;
  t.sg = 1.0f;
  t.hy = t.hx = 0;
  t.by0 = (int)yo * a.sh - a.ph;
  t.bx0 = (int)xo * a.sw - a.pw;

  float acc = 0.0f;
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const Tap q = tap_geometry<DT, MODE, KS>(a, t, om, k);
    TapData<DT, 1, 1> d;
    d.load(xr, q);
    d.accumulate(&acc, q);
  }
  asm volatile("" : "+v"(acc));  // the conversion is its own rounding
  reinterpret_cast<typename io::raw*>(a.y)[(uint64_t)p * (uint32_t)a.C + c] = io::enc(acc);
}


// ------------------------------------------------------------ tiled kernel
// Gathers from an LDS copy of the input instead of from global memory.  On
// MI355X divergent 16-byte global gathers that miss L1 run at about 0.4 cache
// lines per clock per CU, while random 16-byte LDS reads run at about 4.5
// lanes per clock per CU: the workgroup therefore copies, with coalesced
// 128-bit loads, the zero-padded input window its tile can sample (tile
// footprint plus a margin of M pixels on every side) for its chunk of GB
// groups, and the tile's offset/weight values.  A point whose four corners
// lie in the window is gathered from LDS -- corners outside the image read
// the staged zeros, and fma(c, 0, acc) == acc for a finite coefficient.  A
// lane whose point leaves the window, or whose weight is not finite, takes
// the global path of the direct kernel for that point (its wave's other
// lanes stay on LDS).  Both paths perform the same operations on the same values, so the result
// does not depend on which path ran.
typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
// F16W: the window holds the fp16 encoding of the bf16 input (see
// stage_window_f16), so a corner value widens inside the fma (v_fma_mix_f32
// takes an fp16 operand) instead of costing a shift or mask of its own.
template <int DT, int VEC, int NV> struct LdsTap {
  u32x4 v[4][NV];
  // e00, e10: LDS addresses of the even slots of corners (y0, x0) and
  // (y0 + 1, x0); o00, o10 those of the odd slots (the lane's vector order is
  // swapped pairwise or not, see TileLane); dx1: bytes to corner x0 + 1
  __device__ __forceinline__ void load(uint32_t e00, uint32_t e10, uint32_t o00,
                                       uint32_t o10, uint32_t dx1) {
    const uint32_t ea[4] = {e00, e00 + dx1, e10, e10 + dx1};
    const uint32_t oa[4] = {o00, o00 + dx1, o10, o10 + dx1};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int n = 0; n < NV; ++n)
        v[q][n] = *reinterpret_cast<lds_u32x4*>(
            (uintptr_t)(((n & 1) ? oa[q] : ea[q]) + 16 * (n & ~1)));
  }
  template <bool F16W>
  __device__ __forceinline__ void accumulate(float* acc, const float* c) const {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int n = 0; n < NV; ++n)
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          acc[n * VEC + e] = __builtin_fmaf(
              c[q], F16W ? Io<DCN4_F16>::lane(v[q][n], e) : Io<DT>::lane(v[q][n], e),
              acc[n * VEC + e]);
  }
};

// Per-lane state of the tiled kernel's point loop.
// A lane reads its NV 16-byte vectors per corner in the order n ^ r (r = 0
// or 1, fixed per lane; r = 0 when NV is odd): lanes 2^s apart in a wave then
// start on different LDS banks, which removes the two-way bank conflict that
// 32-byte window pixels otherwise give 16 neighbouring lanes.  The lane's
// accumulators follow the same order, and the output store undoes it.
struct TileLane {
  float lane_f;        // LDS address of the lane's even slots at window cell (c, c)
  float row_f, ps_f;   // LDS bytes per window row / pixel
  float ymax, xmax;    // largest corner cell minus c: WSQ-2-c / WW-2-c (square), else WH-2 / WW-2
  float c;             // cell coordinates are taken relative to (c, c)
  uint32_t row_lds, ps;
  uint32_t odd;        // odd slots minus even slots, 16 - 32r (mod 2^32)
};

// One sample point of the tiled kernel.  by/bx: integer base of the point
// relative to window cell (c, c) (exact floats): the grid point in the
// standard modes, the centre in group-scale mode, where gy/gx are the grid
// offsets and sg the lane's group scale (the direct kernel's geometry, so the
// same fp32 operations); returns true when this lane must take the global
// path for this point (nothing accumulated then).  The decision is per lane:
// lanes whose corners lie in the window gather from LDS even when others of
// their wave do not, so a point that leaves the window for a few lanes costs
// global loads for those lanes only.
// SQ: the window is square and c is its centre, so the corner cell is inside
// iff max(|yr|, |xr|) <= ymax; the IEEE maximum propagates NaN, and m*0 is
// NaN exactly when m is not finite, which folds the weight test in.
// whole: the window is the whole image plus its zero border, so a cell
// outside it is not inside the image (the definition of `inside` in
// locate), and its sample adds nothing: that lane skips the point (the
// global path adds fma(0, 0, acc) = acc there, acc never being -0); a
// non-finite weight still sends its lane to the global path, which weights a
// corner outside the image by an exact 0 rather than m * w.
template <int DT, int VEC, int NV, int MODE, int PSC, bool SQ, bool WHOLE, bool F16W>
__device__ __forceinline__ bool tile_point(const TileLane& w,
                                           float by, float bx, float gy, float gx,
                                           float dy, float dx, float m, float os,
                                           float sg, float* acc) {
  const Loc l = sample_location<MODE>(by, bx, gy, gx, dy, dx, os, sg);
  const float fy = __builtin_floorf(l.ty), fx = __builtin_floorf(l.tx);
  const float yr = by + fy, xr = bx + fx;  // corner (y0, x0) minus (c, c)
  bool off_window;
  bool skip = false;
  if constexpr (SQ) {
    const float tc = __builtin_elementwise_maximum(__builtin_fabsf(yr), __builtin_fabsf(xr));
    if constexpr (WHOLE) {
      skip = !(tc <= w.ymax);
      off_window = !__builtin_isfinite(m);
    } else {
      const float t = __builtin_elementwise_maximum(tc, __builtin_fabsf(m * 0.0f));
      off_window = !(t <= w.ymax);
    }
  } else if constexpr (WHOLE) {
    skip = !(yr >= -w.c) || !(yr <= w.ymax) || !(xr >= -w.c) || !(xr <= w.xmax);
    off_window = !__builtin_isfinite(m);
  } else {
    // NaN fails every comparison
    off_window = !(yr >= -w.c) || !(yr <= w.ymax) || !(xr >= -w.c) || !(xr <= w.xmax) ||
                 !__builtin_isfinite(m);
  }
  if (off_window || skip) return off_window;  // skip: outside the image, nothing to add
  const float lh = l.ty - fy, lw = l.tx - fx;
  const float hh = 1.0f - lh, hw = 1.0f - lw;
  const float cf[4] = {m * (hh * hw), m * (hh * lw), m * (lh * hw), m * (lh * lw)};
  // LDS byte address of corner (y0, x0): every term an integer below 2^24,
  // so the fp32 arithmetic is exact
  const uint32_t a00 = (uint32_t)__builtin_fmaf(yr, w.row_f, __builtin_fmaf(xr, w.ps_f, w.lane_f));
  const uint32_t a10 = a00 + w.row_lds;
  LdsTap<DT, VEC, NV> d;
  if (NV > 1)
    d.load(a00, a10, a00 + w.odd, a10 + w.odd, PSC ? (uint32_t)PSC : w.ps);
  else
    d.load(a00, a10, a00, a10, PSC ? (uint32_t)PSC : w.ps);
  d.template accumulate<F16W>(acc, cf);
  return false;
}

// PSC: the LDS bytes per window pixel when known at compile time (one lane
// owns one whole group, no padding, square window), else 0.
// Origin of a tiled workgroup: image, tile, window corner and chunk (a chunk
// is GB whole groups, or one channel slice of one group).  The chunk varies
// fastest in the (XCD-remapped) workgroup order, so the chunks of one tile
// run back to back on one XCD.
struct TileOrigin {
  uint32_t n, g0, s;  // image, first group, channel slice
  int ty0, tx0, wy0, wx0;
};

__device__ __forceinline__ TileOrigin tile_origin(const TileArgs& a) {
  const uint32_t lb = (uint32_t)xcd_block(blockIdx.x, a.nblocks);
  uint32_t q = fastdiv(lb, a.div_chunks);
  const uint32_t gc = lb - q * (uint32_t)a.chunks;
  // chunk gc: group chunk gc / slices, channel slice gc % slices
  const uint32_t gq = fastdiv(gc, a.div_slices);
  uint32_t q2 = fastdiv(q, a.div_tx);
  const uint32_t tx = q - q2 * (uint32_t)a.tiles_x;
  TileOrigin o;
  o.n = fastdiv(q2, a.div_ty);
  const uint32_t ty = q2 - o.n * (uint32_t)a.tiles_y;
  o.ty0 = (int)ty * a.TH * a.passes;
  o.tx0 = (int)tx * a.TW * a.passes_x;
  // the window: the tile's footprint plus the margin, or the whole image and
  // its zero border
  o.wy0 = a.whole ? -1 : o.ty0 * a.sh - a.ph - a.M;
  o.wx0 = a.whole ? -1 : o.tx0 * a.sw - a.pw - a.M;
  o.g0 = gq * (uint32_t)a.GB;
  o.s = gc - gq * (uint32_t)a.slices;
  return o;
}

// Stage the input window of a tile (zeros outside the image) at `lds` in
// passes of wrpp whole window rows.  A window pixel is PS bytes in LDS: its GB
// groups' channels (or the chunk's channel slice), then (when padded) one
// 16-byte chunk loaded as zeros.
// Thread t copies chunk t of every pass, so lane order equals LDS order as
// the global-to-LDS copy requires, and its column, chunk and column test are
// fixed.  Returns the input's buffer descriptor for the image.
template <int es>
__device__ __forceinline__ rsrc_t stage_window(const TileArgs& a, const TileOrigin& o, char* lds) {
  const uint32_t t = threadIdx.x, lane = t & 63u;
  // first thread of the wave, made provably uniform: the LDS destination of
  // a global-to-LDS copy must be, or the compiler loops over its values
  const uint32_t wave0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(t - lane));
  const uint32_t pix_bytes = (uint32_t)(a.C * es);
  const int wy0 = o.wy0, wx0 = o.wx0;
  const uint32_t g0 = o.g0;
  const rsrc_t xr = make_rsrc(a.x + (uint64_t)o.n * a.img_bytes, a.img_bytes);
  {
    const uint32_t cvec = (uint32_t)a.PS >> 4;
    const uint32_t rp = fastdiv(t, a.div_cpr);  // row within the pass
    const uint32_t cc = t - rp * (uint32_t)a.cpr;
    const uint32_t col = fastdiv(cc, a.div_cvec), ch = cc - col * cvec;
    const int gcol = wx0 + (int)col;
    const bool col_ok = ch < ((uint32_t)a.CB >> 4) && (uint32_t)gcol < (uint32_t)a.W;
    const bool copies = rp < (uint32_t)a.wrpp;
    const uint32_t row_bytes = (uint32_t)a.W * pix_bytes;
    int row = wy0 + (int)rp;
    // byte offset of (row, gcol, chunk); used only while it is in the image
    uint32_t off = (uint32_t)row * row_bytes + (uint32_t)gcol * pix_bytes +
                   g0 * (uint32_t)(a.D * es) + o.s * (uint32_t)a.CB + ch * 16u;
    const uint32_t pass_bytes = (uint32_t)a.wrpp * row_bytes;
    const int row_end = wy0 + a.WH;
    char* dst = lds + wave0 * 16u;
    const uint32_t pass_lds = (uint32_t)(a.wrpp * a.cpr) * 16u;
    for (int p = 0; p < a.wpasses; ++p) {
      if (copies && row < row_end) {
        const bool in = col_ok && (uint32_t)row < (uint32_t)a.H;
        copy16_to_lds(xr, dst, in ? off : kOutside);
      }
      row += a.wrpp;
      off += pass_bytes;
      dst += pass_lds;
    }
  }
  return xr;
}

// bf16 -> fp16 re-encoding of the tiled kernel's window.  The inner loop costs
// an fma and a widening per bf16 corner value (a shift or a mask: no gfx950
// fma takes a bf16 operand), but only an fma per fp16 value (v_fma_mix_f32
// widens fp16 inside the fma).  A bf16 value is an fp16 value exactly when it
// is zero or its magnitude lies in [2^-17, 65280]: its exponent is then one of
// fp16's normal exponents or lands on fp16's subnormal grid (steps of 2^-24,
// which the 7 fraction bits of 2^-17 just reach), and its 7 fraction bits fit
// fp16's 10.  The window is restaged as fp16 only when every value of it is
// such a value, so the sum sees the same fp32 operands either way.
constexpr uint32_t kF16MagMax = 0x477fu;   // bf16 magnitude bits of 65280
constexpr uint32_t kF16MagMin1 = 0x36ffu;  // bf16 magnitude bits of 2^-17, minus 1
// Staging passes held in registers.  16 was measured slower: the longer
// unrolled staging costs the U-Net block and the InternImage stage ~1-3 us,
// and FlowDCN's 15-pass fp16 window (margin 5) 102.3 us against 94.6 us
// for its bf16 window copied straight to LDS.
constexpr int kF16WinPasses = 10;
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Two bf16 values (low, high half) to two fp16 values; exact for the values
// above (the rounding mode of the packed conversion never applies).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  const float lo = __uint_as_float(u << 16), hi = __uint_as_float(u & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// stage_window for bf16 windows of at most kF16WinPasses passes, through
// registers: every thread loads its chunks, the workgroup agrees (one word
// per wave at `flags`, 16 bytes of LDS, and a barrier) whether every staged
// value converts exactly, and the window is written to LDS as fp16 if so,
// as the unchanged bf16 bits if not.  Returns true when LDS holds fp16.  The
// window's LDS writes are issued but not waited for: the caller's barrier
// orders them before the first read.
__device__ __forceinline__ bool stage_window_f16(const TileArgs& a, const TileOrigin& o,
                                                 char* lds, rsrc_t xr, char* flags) {
  const uint32_t t = threadIdx.x, lane = t & 63u;
  const uint32_t pix_bytes = (uint32_t)a.C * 2u;
  const uint32_t cvec = (uint32_t)a.PS >> 4;
  const uint32_t rp = fastdiv(t, a.div_cpr);  // row within the pass
  const uint32_t cc = t - rp * (uint32_t)a.cpr;
  const uint32_t col = fastdiv(cc, a.div_cvec), ch = cc - col * cvec;
  const int gcol = o.wx0 + (int)col;
  const bool col_ok = ch < ((uint32_t)a.CB >> 4) && (uint32_t)gcol < (uint32_t)a.W;
  const bool copies = rp < (uint32_t)a.wrpp;
  const uint32_t row_bytes = (uint32_t)a.W * pix_bytes;
  const int row0 = o.wy0 + (int)rp;
  uint32_t off = (uint32_t)row0 * row_bytes + (uint32_t)gcol * pix_bytes +
                 o.g0 * (uint32_t)(a.D * 2) + o.s * (uint32_t)a.CB + ch * 16u;
  const uint32_t pass_bytes = (uint32_t)a.wrpp * row_bytes;
  const int row_end = o.wy0 + a.WH;
  // passes beyond wpasses are skipped by a scalar branch; a lane without a
  // chunk in a pass loads zeros (out-of-range offset) and writes nothing
  u32x4 v[kF16WinPasses];
#pragma unroll
  for (int p = 0; p < kF16WinPasses; ++p) {
    v[p] = (u32x4){0u, 0u, 0u, 0u};
    if (p < a.wpasses) {
      const int row = row0 + p * a.wrpp;
      const bool in = copies && col_ok && row < row_end && (uint32_t)row < (uint32_t)a.H;
      v[p] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(in ? off : kOutside), 0, 0);
    }
    off += pass_bytes;
  }
  // largest magnitude, and smallest magnitude minus one (zero wraps to the
  // largest), per half-word lane of the packed 16-bit operations
  u16x2 mx = {0, 0}, mn = {0xffff, 0xffff};
#pragma unroll
  for (int p = 0; p < kF16WinPasses; ++p) {
    if (p < a.wpasses) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u16x2 m = __builtin_bit_cast(u16x2, v[p][e] & 0x7fff7fffu);
        mx = __builtin_elementwise_max(mx, m);
        mn = __builtin_elementwise_min(mn, m + (u16x2){0xffff, 0xffff});
      }
    }
  }
  const bool ok = (uint32_t)__builtin_elementwise_max(mx.x, mx.y) <= kF16MagMax &&
                  (uint32_t)__builtin_elementwise_min(mn.x, mn.y) >= kF16MagMin1;
  const uint64_t bad = __builtin_amdgcn_ballot_w64(!ok);
  typedef __attribute__((address_space(3))) uint32_t lds_u32;
  if (lane == 0)
    *reinterpret_cast<lds_u32*>((uintptr_t)(__attribute__((address_space(3))) char*)(flags + (t >> 6) * 4u)) =
        bad == 0 ? 1u : 0u;
  __syncthreads();
  const u32x4 f = *reinterpret_cast<lds_u32x4*>(
      (uintptr_t)(__attribute__((address_space(3))) char*)flags);
  const bool f16 = __builtin_amdgcn_readfirstlane((int)(f[0] & f[1] & f[2] & f[3])) != 0;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4_w;
  const uint32_t dst0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds + t * 16u;
  const uint32_t pass_lds = (uint32_t)(a.wrpp * a.cpr) * 16u;
#pragma unroll
  for (int p = 0; p < kF16WinPasses; ++p) {
    if (p < a.wpasses) {
      if (f16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[p][e] = bf16x2_to_f16x2(v[p][e]);
      }
      const int row = row0 + p * a.wrpp;
      if (copies && row < row_end)
        *reinterpret_cast<lds_u32x4_w*>((uintptr_t)(dst0 + (uint32_t)p * pass_lds)) = v[p];
    }
  }
  return f16;
}

// The same re-encoding for a bf16 window already copied to LDS by
// stage_window, for windows of more staging passes than the registers hold:
// every thread reads back the 16-byte chunks it copied, the workgroup agrees
// (as in stage_window_f16) whether every value converts exactly, and if so
// each thread rewrites its chunks as fp16.  Called after a barrier that
// follows the copies; returns true when LDS holds fp16.  The rewrites are
// issued but not waited for: the caller's barrier orders them before the
// first read.
__device__ __forceinline__ bool convert_window_f16(const TileArgs& a, char* lds, char* flags) {
  const uint32_t t = threadIdx.x, lane = t & 63u;
  const uint32_t rp = fastdiv(t, a.div_cpr);  // row within the pass
  const bool copies = rp < (uint32_t)a.wrpp;
  const uint32_t pass_lds = (uint32_t)(a.wrpp * a.cpr) * 16u;
  const uint32_t dst0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds + t * 16u;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4_w;
  u16x2 mx = {0, 0}, mn = {0xffff, 0xffff};
  for (int p = 0; p < a.wpasses; ++p) {
    if (copies && (int)rp + p * a.wrpp < a.WH) {
      const u32x4 v = *reinterpret_cast<lds_u32x4_w*>((uintptr_t)(dst0 + (uint32_t)p * pass_lds));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const u16x2 m = __builtin_bit_cast(u16x2, v[e] & 0x7fff7fffu);
        mx = __builtin_elementwise_max(mx, m);
        mn = __builtin_elementwise_min(mn, m + (u16x2){0xffff, 0xffff});
      }
    }
  }
  const bool ok = (uint32_t)__builtin_elementwise_max(mx.x, mx.y) <= kF16MagMax &&
                  (uint32_t)__builtin_elementwise_min(mn.x, mn.y) >= kF16MagMin1;
  const uint64_t bad = __builtin_amdgcn_ballot_w64(!ok);
  typedef __attribute__((address_space(3))) uint32_t lds_u32;
  if (lane == 0)
    *reinterpret_cast<lds_u32*>((uintptr_t)(__attribute__((address_space(3))) char*)(flags + (t >> 6) * 4u)) =
        bad == 0 ? 1u : 0u;
  __syncthreads();
  const u32x4 f = *reinterpret_cast<lds_u32x4*>(
      (uintptr_t)(__attribute__((address_space(3))) char*)flags);
  const bool f16 = __builtin_amdgcn_readfirstlane((int)(f[0] & f[1] & f[2] & f[3])) != 0;
  if (f16) {
    for (int p = 0; p < a.wpasses; ++p) {
      if (copies && (int)rp + p * a.wrpp < a.WH) {
        lds_u32x4_w* q = reinterpret_cast<lds_u32x4_w*>((uintptr_t)(dst0 + (uint32_t)p * pass_lds));
        u32x4 v = *q;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = bf16x2_to_f16x2(v[e]);
        *q = v;
      }
    }
  }
  return f16;
}

// Stage the tile's offset/weight values at `lds_om`.  Per tile pixel the
// chunk's GB*3K values are OSU units of OMU bytes (4 or 16: fewer copy
// instructions for the larger unit) from the 4-byte boundary at or below their
// start (rows are 4-byte aligned, so the lead `mis`, returned, is the same
// for every pixel); a unit may run into the next chunk's values, which are
// never read.  Passes of orpp whole tile rows when a row's
// units fit the workgroup (thread t then keeps its column and unit), else
// passes of oppp whole pixels.
template <int es>
__device__ __forceinline__ uint32_t stage_om(const TileArgs& a, const TileOrigin& o, int K,
                                             char* lds_om) {
  const uint32_t t = threadIdx.x, lane = t & 63u;
  // first thread of the wave, made provably uniform: the LDS destination of
  // a global-to-LDS copy must be, or the compiler loops over its values
  const uint32_t wave0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(t - lane));
  const int ty0 = o.ty0, tx0 = o.tx0;
  const uint32_t g0 = o.g0;
  const rsrc_t omr = make_rsrc(a.om + (uint64_t)o.n * a.om_img_bytes, a.om_img_bytes);
  const uint32_t seg = g0 * (uint32_t)(3 * K * es);
  const uint32_t mis = seg & 3u;
  const int unit = a.OMU;
  char* om_dst = lds_om + wave0 * (uint32_t)unit;
  if (a.orpp == 1) {
    // one tile row per pass: the row is the same for every copying thread
    const uint32_t upx = fastdiv(t, a.div_osu), e = t - upx * (uint32_t)a.OSU;
    const int xo = tx0 + (int)upx;
    const bool copies = t < (uint32_t)a.upr;
    const bool col_ok = xo < a.Wo;
    uint32_t off = ((uint32_t)ty0 * (uint32_t)a.Wo + (uint32_t)xo) * a.om_row_bytes +
                   (seg - mis) + (uint32_t)unit * e;
    const uint32_t pass_bytes = (uint32_t)a.Wo * a.om_row_bytes;
    const uint32_t pass_lds = (uint32_t)a.upr * (uint32_t)unit;
    const int rows = min(a.TH, a.Ho - ty0);  // rows of the tile inside the output
    for (int p = 0; p < a.TH; ++p) {
      if (copies) {
        const bool in = col_ok && p < rows;
        copy_unit_to_lds(unit, omr, om_dst, in ? off : kOutside);
      }
      off += pass_bytes;
      om_dst += pass_lds;
    }
  } else if (a.orpp > 0) {
    const uint32_t rp = fastdiv(t, a.div_upr);
    const uint32_t u = t - rp * (uint32_t)a.upr;
    const uint32_t upx = fastdiv(u, a.div_osu), e = u - upx * (uint32_t)a.OSU;
    const int xo = tx0 + (int)upx;
    const bool col_ok = xo < a.Wo;
    const bool copies = rp < (uint32_t)a.orpp;
    int yo = ty0 + (int)rp;
    uint32_t off = ((uint32_t)yo * (uint32_t)a.Wo + (uint32_t)xo) * a.om_row_bytes +
                   (seg - mis) + (uint32_t)unit * e;
    const uint32_t pass_bytes = (uint32_t)a.orpp * (uint32_t)a.Wo * a.om_row_bytes;
    const int yo_end = ty0 + a.TH;
    const uint32_t pass_lds = (uint32_t)(a.orpp * a.upr) * (uint32_t)unit;
    for (int p = 0; p < a.opasses; ++p) {
      if (copies && yo < yo_end) {
        const bool in = col_ok && yo < a.Ho;
        copy_unit_to_lds(unit, omr, om_dst, in ? off : kOutside);
      }
      yo += a.orpp;
      off += pass_bytes;
      om_dst += pass_lds;
    }
  } else {
    const uint32_t pp = fastdiv(t, a.div_osu), e = t - pp * (uint32_t)a.OSU;
    const bool copies = pp < (uint32_t)a.oppp;
    const uint32_t npix = (uint32_t)(a.TH * a.TW);
    const uint32_t pass_lds = (uint32_t)(a.oppp * a.OSU) * (uint32_t)unit;
    for (int p = 0; p < a.opasses; ++p) {
      const uint32_t P = (uint32_t)(p * a.oppp) + pp;
      if (copies && P < npix) {
        const uint32_t qy = fastdiv(P, a.div_tw), qx = P - qy * (uint32_t)a.TW;
        const int yo = ty0 + (int)qy, xo = tx0 + (int)qx;
        const bool in = yo < a.Ho && xo < a.Wo;
        const uint32_t off = ((uint32_t)yo * (uint32_t)a.Wo + (uint32_t)xo) * a.om_row_bytes +
                             (seg - mis) + (uint32_t)unit * e;
        copy_unit_to_lds(unit, omr, om_dst, in ? off : kOutside);
      }
      om_dst += pass_lds;
    }
  }
  return mis;
}

// Words of a 3x3 kernel's offset/weight row held in registers: 27 16-bit
// values from the 4-byte boundary at or below the row (56 bytes), or 27
// fp32 values.
template <int es> constexpr int kOmWords = es == 2 ? 14 : 27;

// Value j of a lane's offset/weight row held in registers: w holds the row
// from a 4-byte boundary; with 16-bit values P = 1 when the row starts at an
// odd 16-bit position (a group's row of 3K values, K odd, is 2-byte aligned
// every other group).
template <int DT, int P>
__device__ __forceinline__ float om_packed(const uint32_t* w, int j) {
  if constexpr (DT == DCN4_F32) {
    return __uint_as_float(w[j]);
  } else {
    const int h = j + P;
    const uint32_t v = w[h >> 1];
    if constexpr (DT == DCN4_BF16)
      return __uint_as_float((h & 1) ? (v & 0xffff0000u) : (v << 16));
    else
      return Io<DT>::dec((typename Io<DT>::raw)((h & 1) ? (v >> 16) : (v & 0xffffu)));
  }
}

// A lane's offset/weight row of a 3x3 kernel read from global memory into
// registers: kOmWords words from the 4-byte boundary at or below the row of
// group g0 at the lane's tile pixel (one group per workgroup); a pixel
// outside the output reads zeros.
template <int es>
__device__ __forceinline__ void load_om_row(const TileArgs& a, uint32_t n, uint32_t g0, int ty0,
                                            int tx0, uint32_t* w) {
  constexpr int words = kOmWords<es>;
  const uint32_t t = threadIdx.x;
  const uint32_t tp = fastdiv(t, a.div_gbl);
  const uint32_t py = fastdiv(tp, a.div_tw), px = tp - py * (uint32_t)a.TW;
  const int yo = ty0 + (int)py, xo = tx0 + (int)px;
  const rsrc_t omr = make_rsrc(a.om + (uint64_t)n * a.om_img_bytes, a.om_img_bytes);
  const uint32_t seg = g0 * (uint32_t)(27 * es);
  const uint32_t off = (yo < a.Ho && xo < a.Wo)
                           ? ((uint32_t)yo * (uint32_t)a.Wo + (uint32_t)xo) * a.om_row_bytes +
                                 (seg & ~3u)
                           : kOutside;
#pragma unroll
  for (int q = 0; q < words / 4; ++q) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(omr, (int)(off + 16u * q), 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[4 * q + e] = v[e];
  }
  constexpr int q4 = words / 4 * 4;
  if constexpr (words - q4 >= 2) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(omr, (int)(off + 4u * q4), 0, 0);
    w[q4] = v[0];
    w[q4 + 1] = v[1];
  }
  if constexpr ((words - q4) % 2)
    w[words - 1] = __builtin_amdgcn_raw_buffer_load_b32(omr, (int)(off + 4u * (words - 1)), 0, 0);
}

// The point loop of the tiled kernel: every point of the lane from LDS, or
// from global memory for a wave with a point outside the window.  F16W: the
// window holds fp16 (see stage_window_f16).
template <int DT, int VEC, int NV, int MODE, int KS, int PSC, bool WHOLE, bool F16W, int OMP>
__device__ __forceinline__ void tile_points(const TileArgs& a, const FwdArgs& fa,
                                            const LaneCtx& c, const TileLane& w,
                                            const typename Io<DT>::raw* om, const uint32_t* omw,
                                            rsrc_t xr, uint32_t r16, float ry0, float rx0,
                                            float* acc) {
  typedef Io<DT> io;
  const int K = KS ? KS * KS : a.kh * a.kw;
  constexpr bool SQ = PSC != 0;
  constexpr bool GS = MODE == kGroupScale;
  if (KS) {
    float bx[KS ? KS : 1];
#pragma unroll
    for (int j = 0; j < KS; ++j) bx[j] = GS ? rx0 : rx0 + (float)(j * a.dw);
    const float fdh = GS ? 0.0f : (float)a.dh;
    float by = ry0;
#pragma unroll
    for (int i = 0; i < KS; ++i, by += fdh) {
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const int k = i * KS + j;
        float dx, dy, m;
        if constexpr (OMP > 0) {
          dx = om_packed<DT, OMP - 1>(omw, 2 * k);
          dy = om_packed<DT, OMP - 1>(omw, 2 * k + 1);
          m = om_packed<DT, OMP - 1>(omw, 2 * K + k);
        } else {
          dx = io::dec(om[2 * k]);
          dy = io::dec(om[2 * k + 1]);
          m = io::dec(om[2 * K + k]);
        }
        const float gyy = GS ? (float)(i - c.hy) : 0.0f, gxx = GS ? (float)(j - c.hx) : 0.0f;
        if (tile_point<DT, VEC, NV, MODE, PSC, SQ, WHOLE, F16W>(w, by, bx[j], gyy, gxx, dy, dx,
                                                          m, a.offset_scale, c.sg, acc)) {
          const Tap tg = tap_geometry_v<MODE, KS>(fa, c, dx, dy, m, k);
          TapData<DT, VEC, NV> d;
          d.load_swapped(xr, tg, r16);
          d.accumulate(acc, tg);
        }
      }
    }
  } else {
    const int kw = a.kw;
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
      const int i = k / kw, j = k - (k / kw) * kw;
      const float dx = io::dec(om[2 * k]);
      const float dy = io::dec(om[2 * k + 1]);
      const float m = io::dec(om[2 * K + k]);
      const float by = GS ? ry0 : ry0 + (float)(i * a.dh);
      const float bx = GS ? rx0 : rx0 + (float)(j * a.dw);
      const float gyy = GS ? (float)(i - c.hy) : 0.0f, gxx = GS ? (float)(j - c.hx) : 0.0f;
      if (tile_point<DT, VEC, NV, MODE, PSC, SQ, WHOLE, F16W>(w, by, bx, gyy, gxx, dy, dx, m,
                                                        a.offset_scale, c.sg, acc)) {
        const Tap tg = tap_geometry<DT, MODE, KS>(fa, c, om, k);
        TapData<DT, VEC, NV> d;
        d.load_swapped(xr, tg, r16);
        d.accumulate(acc, tg);
      }
    }
  }
}

// Occupancy hint of the tiled forward for lanes of at most two vectors
// (a build-time knob): 4 waves per SIMD fit its registers without spills;
// 5 and 6 measured 28-100% slower on the U-Net block, 2 and 3 the same.
#ifndef DCN4_TILE_WAVES_NV2
#define DCN4_TILE_WAVES_NV2 4
#endif
template <int DT, int VEC, int NV, int MODE, int KS, int PSC, bool WHOLE>
__global__ __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(NV <= 2 ? DCN4_TILE_WAVES_NV2 : (NV == 3 ? 3 : 2))))
void dcn4_tile_kernel(TileArgs a) {
  typedef Io<DT> io;
  constexpr int es = io::es;
  constexpr int DP = VEC * NV;
  extern __shared__ u32x4 lds_u4[];
  char* lds = reinterpret_cast<char*>(lds_u4);

  const TileOrigin org = tile_origin(a);
  const uint32_t n = org.n, g0 = org.g0;
  const int wy0 = org.wy0, wx0 = org.wx0;
  const int K = KS ? KS * KS : a.kh * a.kw;
  const uint32_t t = threadIdx.x, lane = t & 63u;
  const uint32_t pix_bytes = (uint32_t)(a.C * es);

  // the offset/weight copies are requested first, so that their latency
  // overlaps the window's (both are waited for at the barriers below)
  constexpr bool PK = KS == 3;
  uint32_t omw[kOmWords<es>];
  const bool omd = PK && a.om_direct;
  uint32_t mis;
  if (PK && omd) {
    mis = (org.g0 * (uint32_t)(27 * es)) & 3u;
    load_om_row<es>(a, org.n, org.g0, org.ty0, org.tx0, omw);
  } else {
    mis = stage_om<es>(a, org, K, lds + a.om_lds);
  }
  // bf16 windows of few enough passes go through registers and become fp16
  // when every value converts exactly (stage_window_f16)
  bool f16w = false;
  rsrc_t xr;
  if constexpr (DT == DCN4_BF16) {
    if (a.f16_window == 1) {
      xr = make_rsrc(a.x + (uint64_t)org.n * a.img_bytes, a.img_bytes);
      f16w = stage_window_f16(a, org, lds, xr, lds + a.flag_lds);
    } else {
      xr = stage_window<es>(a, org, lds);
      if (a.f16_window == 2) {  // re-encoded in LDS after the copies land
        __syncthreads();
        f16w = convert_window_f16(a, lds, lds + a.flag_lds);
      }
    }
  } else {
    xr = stage_window<es>(a, org, lds);
  }
  __syncthreads();

  // A block of `passes` tile rows by `passes_x` tile columns (columns only
  // under the whole-image window) shares one staging of the window (the
  // whole image, or the rows' footprints plus the margin), each pass
  // restaging only the offset/weight rows; columns vary fastest.
  const int npass = a.passes * a.passes_x;
  for (int pass = 0; pass < npass; ++pass) {
    const int prow = pass / a.passes_x, pcol = pass - prow * a.passes_x;  // uniform
    const int ty0 = org.ty0 + prow * a.TH, tx0 = org.tx0 + pcol * a.TW;
    if (pass > 0) {
      if (PK && omd) {
        load_om_row<es>(a, org.n, org.g0, ty0, tx0, omw);
      } else {
        __syncthreads();  // every lane is done with the previous rows' offsets
        TileOrigin op = org;
        op.ty0 = ty0;
        op.tx0 = tx0;
        stage_om<es>(a, op, K, lds + a.om_lds);
        __syncthreads();
      }
    }
    // ---- lane -> (tile pixel, group in chunk, channel slice)
    const uint32_t tp = fastdiv(t, a.div_gbl);
    const uint32_t rr = t - tp * (uint32_t)(a.GB * a.L);
    const uint32_t gl = fastdiv(rr, a.div_L), l = rr - gl * (uint32_t)a.L;
    const uint32_t py = fastdiv(tp, a.div_tw), px = tp - py * (uint32_t)a.TW;
    const int yo = ty0 + (int)py, xo = tx0 + (int)px;
    if (yo >= a.Ho || xo >= a.Wo) continue;  // this pass has no output here
    const uint32_t g = g0 + gl;
    const typename io::raw* om = reinterpret_cast<const typename io::raw*>(
        lds + a.om_lds + tp * (uint32_t)(a.OSU * a.OMU) + mis + gl * (uint32_t)(3 * K * es));
    // first channel of the lane within the pixel: its group, slice and lane
    const uint32_t chan = g * (uint32_t)a.D + org.s * (uint32_t)a.DSL + l * DP;

    FwdArgs fa{};  // the geometry reads only the fields FwdArgs and TileArgs share
    fa.H = a.H; fa.W = a.W; fa.G = a.G; fa.kh = a.kh; fa.kw = a.kw; fa.dh = a.dh; fa.dw = a.dw;
    fa.offset_scale = a.offset_scale; fa.Hm1 = a.Hm1; fa.Wm1 = a.Wm1;
    fa.scales = a.scales; fa.pscales = a.pscales; fa.max_scale = a.max_scale;
    // global-path context (points whose corners leave the window)
    LaneCtx c;
    c.pix_bytes = pix_bytes;
    c.row_stride = (uint32_t)a.W * pix_bytes;
    c.lane_bytes = chan * es;
    c.hy = ((KS ? KS : a.kh) - 1) >> 1;
    c.hx = ((KS ? KS : a.kw) - 1) >> 1;
    // group-scale mode: the lane's scale (pixel counted from the launch's first
    // image) and the point base at the centre
    c.sg = (MODE == kGroupScale)
               ? group_scale(fa, ((uint64_t)n * a.Ho + (uint32_t)yo) * a.Wo + (uint32_t)xo, g)
               : 1.0f;
    c.by0 = yo * a.sh - a.ph + (MODE == kGroupScale ? c.hy : 0);
    c.bx0 = xo * a.sw - a.pw + (MODE == kGroupScale ? c.hx : 0);

    TileLane w;
    w.row_lds = (uint32_t)(a.WW * a.PS);
    w.ps = (uint32_t)a.PS;
    w.row_f = (float)w.row_lds;
    w.ps_f = (float)a.PS;
    // the window starts at the LDS allocation's base address
    const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
    const uint32_t r16 = (NV % 2 == 0 && a.swz_shift >= 0) ? ((lane >> a.swz_shift) & 1u) * 16u : 0u;
    w.lane_f = (float)(lds_base + (gl * (uint32_t)a.D + l * DP) * es + r16);
    w.odd = 16u - 2u * r16;
    // cell coordinates relative to (cy, cw): the centre of a square window
    // (with margin-window passes, of the square WSQ rows high that this
    // pass's tile row alone would stage, pass * TH * sh rows down)
    constexpr bool SQ = PSC != 0;
    const float cw = SQ ? 0.5f * (float)(a.WSQ - 2) : 0.0f;
    const float cy = (SQ && !WHOLE) ? cw + (float)(prow * a.TH * a.sh) : cw;
    w.c = cw;
    w.ymax = SQ ? (float)(a.WSQ - 2) - cw : (float)(a.WH - 2);
    w.xmax = (float)(a.WW - 2) - cw;
    w.lane_f += cy * w.row_f + cw * w.ps_f;  // exact: small multiples of 1/2
    // base of point (0, 0) relative to window cell (cy, cw)
    const float ry0 = (float)(c.by0 - wy0) - cy, rx0 = (float)(c.bx0 - wx0) - cw;

    float acc[DP];
#pragma unroll
    for (int e = 0; e < DP; ++e) acc[e] = 0.0f;

    // 16-bit offset/weight rows of a 3x3 kernel, one group per workgroup: the
    // lane's 27 values are read up front as seven 8-byte words (the row
    // start is 8-byte aligned: tile pixels are OSU*OMU bytes apart, a
    // multiple of 8 here) instead of one 2-byte read before each point
    const bool pk = PK && (omd || (es == 2 && a.GB == 1 && ((a.OSU * a.OMU) & 7) == 0));
    if (PK && es == 2 && pk && !omd) {
      typedef const __attribute__((address_space(3))) uint64_t lds_u64;
      const uint32_t b = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(
                             reinterpret_cast<const char*>(om) - mis);
#pragma unroll
      for (int q = 0; q < 7; ++q) {
        const uint64_t v = *reinterpret_cast<lds_u64*>((uintptr_t)(b + 8u * q));
        omw[2 * q] = (uint32_t)v;
        omw[2 * q + 1] = (uint32_t)(v >> 32);
      }
    }
    if constexpr (DT == DCN4_BF16) {
      if (f16w) {
        if (PK && pk && mis)
          tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, true, 2>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
        else if (PK && pk)
          tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, true, 1>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
        else
          tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, true, 0>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
      } else {
        if (PK && pk && mis)
          tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, false, 2>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
        else if (PK && pk)
          tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, false, 1>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
        else
          tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, false, 0>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
      }
    } else if constexpr (PK) {
      if (es == 2 && pk && mis)
        tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, false, (es == 2 ? 2 : 1)>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
      else if (pk)
        tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, false, 1>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
      else
        tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, false, 0>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
    } else {
      tile_points<DT, VEC, NV, MODE, KS, PSC, WHOLE, false, 0>(a, fa, c, w, om, omw, xr, r16, ry0, rx0, acc);
    }

#pragma unroll
    for (int e = 0; e < DP; ++e) asm volatile("" : "+v"(acc[e]));
    char* yp = a.y + (((uint64_t)n * a.Ho + yo) * a.Wo + xo) * pix_bytes + chan * es;
    char* ype = yp + r16;           // even slots
    char* ypo = yp + (16u - r16);   // odd slots
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      u32x4 o;
      if constexpr (es == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(acc[v * VEC + e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = io::enc2(acc[v * VEC + 2 * e], acc[v * VEC + 2 * e + 1]);
      }
      *reinterpret_cast<u32x4*>(((v & 1) ? ypo : ype) + 16 * (v & ~1)) = o;
    }
  }
}

// ------------------------------------------------------------ backward
// Gradients of the forward pass for an upstream gradient gy (fp32 results):
//   grad_x[corner, c] += m_k * w_corner * gy[p, c]      (scatter, fp32 atomics)
//   grad_m[p, g, k]    = sum_c gy[p, c] * B_c
//   grad_d{y,x}[p,g,k] = m_k * f * sum_c gy[p, c] * dB_c/d{row,col}
// with B the bilinear sample, f = offset_scale or the group's scale, and, in
// the cell (y0, x0) with fractions (lh, lw), dB/drow = (1-lw)(v10-v00) +
// lw(v11-v01), dB/dcol = (1-lh)(v01-v00) + lh(v11-v10).  The sampling
// decisions (cell, fractions, inside test, scale) come from the forward's
// device functions, so they are the forward's bit for bit; a sample that is
// not inside has zero gradient.
// All three are linear in the corner values, so the kernels first sum
// S_r = sum_c gy[p, c] * v_r,c per corner r (one fma per channel and corner)
// and then combine the four sums (point_grads); every term of the
// definitions above still enters once, with its own fp32 rounding.
//
// Lanes: Lg lanes per (pixel, group) item, lane li owning channels li,
// li + Lg, ... of the group (Lg = the largest power of two <= 16 dividing D).
// For one channel index the Lg lanes of an item touch Lg consecutive
// channels, so a wave's atomics and gathers cover 64/Lg contiguous runs of
// Lg elements rather than 64 scattered cache lines.  The three per-point
// reductions over the group's channels are xor-shuffles within the item.
struct BwdArgs {
  const char* x;          // input of this launch's first image
  const char* om;         // offset/weight tensor of this launch's first image
  const float* scales;
  const float* pscales;   // [pixels, G] of this launch, or null
  const char* gy;         // upstream gradient [N,Ho,Wo,C], I/O dtype
  float* gx;              // [N,H,W,C] fp32 (accumulated), or null
  float* gom;             // [N,Ho,Wo,G,3K] fp32 (written), or null
  FwdArgs f;              // geometry fields shared with the forward
  int32_t lg_shift;       // log2(Lg)
  int64_t lanes;          // lanes of this launch
  uint64_t x_bytes;       // input bytes of this launch
  int32_t nvec;           // vector kernel: 16-byte vectors per group, D*es/16
};

// The point's three gradient sums from its corner sums S (order 00, 01, 10,
// 11), bilinear weights w and fractions: sum_c gy*B, sum_c gy*dB/drow,
// sum_c gy*dB/dcol (the latter two before the factor m*f).
__device__ __forceinline__ void point_grads(const float* S, const float* w, float lh, float lw,
                                            float& gm, float& gdr, float& gdc) {
  const float hh = 1.0f - lh, hw = 1.0f - lw;
  gm = w[0] * S[0];
  gm = __builtin_fmaf(w[1], S[1], gm);
  gm = __builtin_fmaf(w[2], S[2], gm);
  gm = __builtin_fmaf(w[3], S[3], gm);
  gdr = __builtin_fmaf(lw, S[3] - S[1], hw * (S[2] - S[0]));
  gdc = __builtin_fmaf(lh, S[3] - S[2], hh * (S[1] - S[0]));
}

template <int DT, int MODE, int KS>
__global__ __launch_bounds__(kBlock) void dcn4_backward_kernel(BwdArgs b) {
  typedef Io<DT> io;
  constexpr int es = io::es;
  const FwdArgs& a = b.f;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (gid >= b.lanes) return;
  const int Lg = 1 << b.lg_shift;
  const uint32_t item = (uint32_t)(gid >> b.lg_shift);
  const uint32_t li = (uint32_t)gid & (uint32_t)(Lg - 1);
  const uint32_t p = fastdiv(item, a.div_ipp);  // ipp = G here
  const uint32_t g = item - p * (uint32_t)a.G;
  const uint32_t n = fastdiv(p, a.div_hw);
  const uint32_t rem = p - n * (uint32_t)(a.Ho * a.Wo);
  const uint32_t yo = fastdiv(rem, a.div_wo);
  const uint32_t xo = rem - yo * (uint32_t)a.Wo;
  const int K = KS ? KS * KS : a.kh * a.kw;
  const int kw = KS ? KS : a.kw;
  const int cpl = a.D >> b.lg_shift;  // channels per lane

  const typename io::raw* om = reinterpret_cast<const typename io::raw*>(b.om) +
                               (uint64_t)item * (uint32_t)(3 * K);
  const typename io::raw* gyp = reinterpret_cast<const typename io::raw*>(b.gy) +
                                (uint64_t)p * (uint32_t)a.C + g * (uint32_t)a.D + li;
  const rsrc_t xr = make_rsrc(b.x, (uint32_t)(b.x_bytes < 0x7fffffffu ? b.x_bytes : 0x7fffffffu));
  const uint32_t pix_bytes = (uint32_t)a.C * es;
  const uint32_t img_off = n * a.img_bytes + (g * (uint32_t)a.D + li) * es;
  float* gxp = b.gx ? b.gx + (uint64_t)n * a.H * a.W * a.C + g * (uint32_t)a.D + li : nullptr;
  const float sg = (MODE == kGroupScale) ? group_scale(a, p, g) : 1.0f;
  const float f = (MODE == kGroupScale) ? sg : a.offset_scale;
  const int hy = ((KS ? KS : a.kh) - 1) >> 1, hx = (kw - 1) >> 1;

#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const int i = k / kw, j = k - (k / kw) * kw;
    const float dx = io::dec(om[2 * k]);
    const float dy = io::dec(om[2 * k + 1]);
    const float m = io::dec(om[2 * K + k]);
    float by, bx, gyy = 0.0f, gxx = 0.0f;
    if (MODE == kGroupScale) {
      by = (float)((int)yo * a.sh - a.ph + hy);
      bx = (float)((int)xo * a.sw - a.pw + hx);
      gyy = (float)(i - hy);
      gxx = (float)(j - hx);
    } else {
      by = (float)((int)yo * a.sh - a.ph + i * a.dh);
      bx = (float)((int)xo * a.sw - a.pw + j * a.dw);
    }
    const Cell c = locate(sample_location<MODE>(by, bx, gyy, gxx, dy, dx, a.offset_scale, sg),
                          a.Hm1, a.Wm1);
    float gm = 0.0f, gdr = 0.0f, gdc = 0.0f;
    if (c.inside) {
      const bool vy0 = c.y0 >= 0, vy1 = c.y0 < a.H - 1;
      const bool vx0 = c.x0 >= 0, vx1 = c.x0 < a.W - 1;
      const bool ok[4] = {vy0 && vx0, vy0 && vx1, vy1 && vx0, vy1 && vx1};
      const float lh = c.lh, lw = c.lw, hh = 1.0f - lh, hw = 1.0f - lw;
      const float w[4] = {hh * hw, hh * lw, lh * hw, lh * lw};
      const int cy[4] = {c.y0, c.y0, c.y0 + 1, c.y0 + 1};
      const int cx[4] = {c.x0, c.x0 + 1, c.x0, c.x0 + 1};
      uint32_t q[4];
      float cm[4];
      float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // corner sums of gy * v
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // pixel index below 2^23 (H*W < 2^23); only used for corners in the image
        const uint32_t pix = (uint32_t)(cy[r] * a.W + cx[r]);
        q[r] = ok[r] ? img_off + pix * pix_bytes : kOutside;
        cm[r] = m * w[r];
      }
#pragma unroll 1
      for (int jc = 0; jc < cpl; ++jc) {
        const uint32_t coff = ((uint32_t)jc << b.lg_shift) * es;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (es == 4)
            v[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, (int)(q[r] + coff), 0, 0));
          else
            v[r] = io::dec((typename io::raw)__builtin_amdgcn_raw_buffer_load_b16(xr, (int)(q[r] + coff), 0, 0));
        }
        const float gyc = io::dec(gyp[jc << b.lg_shift]);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[r] = __builtin_fmaf(gyc, v[r], S[r]);
        if (gxp) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (ok[r])
              unsafeAtomicAdd(gxp + ((uint64_t)(cy[r] * a.W + cx[r]) * (uint32_t)a.C +
                                     ((uint32_t)jc << b.lg_shift)),
                              cm[r] * gyc);
        }
      }
      point_grads(S, w, lh, lw, gm, gdr, gdc);
    }
    if (b.gom) {
      // the item's Lg lanes are consecutive and Lg-aligned in the wave
      for (int off = 1; off < Lg; off <<= 1) {
        gm += __shfl_xor(gm, off, 64);
        gdr += __shfl_xor(gdr, off, 64);
        gdc += __shfl_xor(gdc, off, 64);
      }
      if (li == 0) {
        float* go = b.gom + (uint64_t)item * (uint32_t)(3 * K);
        const float mf = m * f;
        go[2 * k] = mf * gdc;      // dx moves the column
        go[2 * k + 1] = mf * gdr;  // dy moves the row
        go[2 * K + k] = gm;
      }
    }
  }
}

// Gradients of FlowDCN's scales (group-scale mode).  Point k of the item's
// group samples centre + S * u_k on each axis, u_k = fl(grid_k + d_k) the
// value sample_location multiplies by the effective scale S, so
//   dL/dS = sum_k m_k * (u_y,k * sum_c gy dB/drow + u_x,k * sum_c gy dB/dcol)
// over the inside samples (the forward's sampling decisions); below the clamp
// S = s_g * sigma, so dL/dsigma = s_g * dL/dS and dL/ds_g sums sigma * dL/dS
// over the pixels; above it (fl(s_g * sigma) > Smax) both are 0.  Lanes as in
// dcn4_backward_kernel: Lg channel-strided lanes per (pixel, group) item, each
// with its partial sums over its channels; the item's lanes are added by
// xor-shuffles, the items of a workgroup per group in LDS, and the workgroup
// adds one fp32 atomic per group into gsg (cleared by the launcher), so
// dL/ds_g is summed in no fixed order.
template <int DT, int KS>
__global__ __launch_bounds__(kBlock) void dcn4_scale_grad_kernel(BwdArgs b, float* gsg,
                                                                 float* gps) {
  typedef Io<DT> io;
  constexpr int es = io::es;
  extern __shared__ float g_lds[];  // [G] per-group partial sums of the workgroup
  const FwdArgs& a = b.f;
  for (uint32_t e = threadIdx.x; e < (uint32_t)a.G; e += kBlock) g_lds[e] = 0.0f;
  __syncthreads();
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const bool active = gid < b.lanes;
  const int Lg = 1 << b.lg_shift;
  const uint32_t item = (uint32_t)((active ? gid : 0) >> b.lg_shift);
  const uint32_t li = (uint32_t)threadIdx.x & (uint32_t)(Lg - 1);
  const uint32_t p = fastdiv(item, a.div_ipp);  // ipp = G here
  const uint32_t g = item - p * (uint32_t)a.G;
  const uint32_t n = fastdiv(p, a.div_hw);
  const uint32_t rem = p - n * (uint32_t)(a.Ho * a.Wo);
  const uint32_t yo = fastdiv(rem, a.div_wo);
  const uint32_t xo = rem - yo * (uint32_t)a.Wo;
  const int K = KS ? KS * KS : a.kh * a.kw;
  const int kw = KS ? KS : a.kw;
  const int cpl = a.D >> b.lg_shift;  // channels per lane
  const typename io::raw* om = reinterpret_cast<const typename io::raw*>(b.om) +
                               (uint64_t)item * (uint32_t)(3 * K);
  const typename io::raw* gyp = reinterpret_cast<const typename io::raw*>(b.gy) +
                                (uint64_t)p * (uint32_t)a.C + g * (uint32_t)a.D + li;
  const rsrc_t xr = make_rsrc(b.x, (uint32_t)(b.x_bytes < 0x7fffffffu ? b.x_bytes : 0x7fffffffu));
  const uint32_t pix_bytes = (uint32_t)a.C * es;
  const uint32_t img_off = n * a.img_bytes + (g * (uint32_t)a.D + li) * es;
  const float sg = group_scale(a, p, g);
  const int hy = ((KS ? KS : a.kh) - 1) >> 1, hx = (kw - 1) >> 1;
  float dS = 0.0f;  // this lane's part of dL/dS
  if (active) {
#pragma unroll 1
    for (int k = 0; k < K; ++k) {
      const int i = k / kw, j = k - (k / kw) * kw;
      const float dx = io::dec(om[2 * k]);
      const float dy = io::dec(om[2 * k + 1]);
      const float m = io::dec(om[2 * K + k]);
      const float gyy = (float)(i - hy), gxx = (float)(j - hx);
      const Cell c = locate(sample_location<kGroupScale>((float)((int)yo * a.sh - a.ph + hy),
                                                         (float)((int)xo * a.sw - a.pw + hx),
                                                         gyy, gxx, dy, dx, a.offset_scale, sg),
                            a.Hm1, a.Wm1);
      if (!c.inside) continue;
      const bool vy0 = c.y0 >= 0, vy1 = c.y0 < a.H - 1;
      const bool vx0 = c.x0 >= 0, vx1 = c.x0 < a.W - 1;
      const bool ok[4] = {vy0 && vx0, vy0 && vx1, vy1 && vx0, vy1 && vx1};
      const float lh = c.lh, lw = c.lw, hh = 1.0f - lh, hw = 1.0f - lw;
      const float w[4] = {hh * hw, hh * lw, lh * hw, lh * lw};
      const int cy[4] = {c.y0, c.y0, c.y0 + 1, c.y0 + 1};
      const int cx[4] = {c.x0, c.x0 + 1, c.x0, c.x0 + 1};
      uint32_t q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        q[r] = ok[r] ? img_off + (uint32_t)(cy[r] * a.W + cx[r]) * pix_bytes : kOutside;
      float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // corner sums of gy * v
#pragma unroll 1
      for (int jc = 0; jc < cpl; ++jc) {
        const uint32_t coff = ((uint32_t)jc << b.lg_shift) * es;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (es == 4)
            v[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, (int)(q[r] + coff), 0, 0));
          else
            v[r] = io::dec((typename io::raw)__builtin_amdgcn_raw_buffer_load_b16(xr, (int)(q[r] + coff), 0, 0));
        }
        const float gyc = io::dec(gyp[jc << b.lg_shift]);
#pragma unroll
        for (int r = 0; r < 4; ++r) S[r] = __builtin_fmaf(gyc, v[r], S[r]);
      }
      float gm, gdr, gdc;
      point_grads(S, w, lh, lw, gm, gdr, gdc);
      // u = grid + direction, the same fp32 sums sample_location scales
      dS = __builtin_fmaf(m, __builtin_fmaf(gyy + dy, gdr, (gxx + dx) * gdc), dS);
    }
  }
  // the item's Lg lanes are consecutive and Lg-aligned in the wave
  for (int off = 1; off < Lg; off <<= 1) dS += __shfl_xor(dS, off, 64);
  if (active && li == 0) {
    float Su = a.scales[g];
    const float sig = a.pscales ? a.pscales[(uint64_t)p * (uint32_t)a.G + g] : 1.0f;
    if (a.pscales) Su = Su * sig;
    if (a.max_scale > 0.0f && Su > a.max_scale) dS = 0.0f;  // S is the constant Smax
    if (gps) gps[(uint64_t)p * (uint32_t)a.G + g] = a.scales[g] * dS;
    if (gsg) atomicAdd(&g_lds[g], sig * dS);
  }
  if (!gsg) return;
  __syncthreads();
  for (uint32_t e = threadIdx.x; e < (uint32_t)a.G; e += kBlock) {
    const float v = g_lds[e];
    if (v != 0.0f) unsafeAtomicAdd(gsg + e, v);
  }
}

// grad_offset_mask alone (grad_x gathered or not asked for) where the tiled
// kernel does not apply, for groups of whole 16-byte vectors and 16-byte
// aligned tensors: Lg lanes per (pixel, group) item, lane li owning the
// group's vectors li, li + Lg, ...; per point one 16-byte corner load per
// vector (zero outside, via the buffer range check), grad_y loaded once per
// item; the three sums of the item reduced by xor-shuffles.  The item's row
// of 3K values collects in LDS; a workgroup's items are consecutive, so
// their rows are one contiguous block of the tensor, stored with consecutive
// threads on consecutive floats.  Sampling decisions and the per-channel
// arithmetic are those of dcn4_backward_kernel (channels summed in another
// order).
template <int DT, int MODE, int KS>
__global__ __launch_bounds__(kBlock) void dcn4_backward_om_kernel(BwdArgs b) {
  typedef Io<DT> io;
  constexpr int es = io::es;
  constexpr int V = 16 / es;
  extern __shared__ float om_rows[];  // [kBlock >> lg_shift][3K]
  const FwdArgs& a = b.f;
  const int64_t gid = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  const bool active = gid < b.lanes;
  const int Lg = 1 << b.lg_shift;
  const uint32_t item = (uint32_t)((active ? gid : 0) >> b.lg_shift);
  const uint32_t li = (uint32_t)threadIdx.x & (uint32_t)(Lg - 1);
  const uint32_t p = fastdiv(item, a.div_ipp);  // ipp = G here
  const uint32_t g = item - p * (uint32_t)a.G;
  const uint32_t n = fastdiv(p, a.div_hw);
  const uint32_t rem = p - n * (uint32_t)(a.Ho * a.Wo);
  const uint32_t yo = fastdiv(rem, a.div_wo);
  const uint32_t xo = rem - yo * (uint32_t)a.Wo;
  const int K = KS ? KS * KS : a.kh * a.kw;
  const int kw = KS ? KS : a.kw;
  const typename io::raw* om = reinterpret_cast<const typename io::raw*>(b.om) +
                               (uint64_t)item * (uint32_t)(3 * K);
  const rsrc_t xr = make_rsrc(b.x, (uint32_t)(b.x_bytes < 0x7fffffffu ? b.x_bytes : 0x7fffffffu));
  const uint32_t pix_bytes = (uint32_t)a.C * es;
  const uint32_t img_off = n * a.img_bytes + g * (uint32_t)(a.D * es);
  const char* gyp = b.gy + ((uint64_t)p * (uint32_t)a.C + g * (uint32_t)a.D) * es;
  const float sg = (MODE == kGroupScale) ? group_scale(a, p, g) : 1.0f;
  const float f = (MODE == kGroupScale) ? sg : a.offset_scale;
  const int hy = ((KS ? KS : a.kh) - 1) >> 1, hx = (kw - 1) >> 1;
  const uint32_t row0 = threadIdx.x >> b.lg_shift;  // the item's row in this workgroup

#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const int i = k / kw, j = k - (k / kw) * kw;
    const float dx = io::dec(om[2 * k]);
    const float dy = io::dec(om[2 * k + 1]);
    const float m = io::dec(om[2 * K + k]);
    float by, bx, gyy = 0.0f, gxx = 0.0f;
    if (MODE == kGroupScale) {
      by = (float)((int)yo * a.sh - a.ph + hy);
      bx = (float)((int)xo * a.sw - a.pw + hx);
      gyy = (float)(i - hy);
      gxx = (float)(j - hx);
    } else {
      by = (float)((int)yo * a.sh - a.ph + i * a.dh);
      bx = (float)((int)xo * a.sw - a.pw + j * a.dw);
    }
    const Cell c = locate(sample_location<MODE>(by, bx, gyy, gxx, dy, dx, a.offset_scale, sg),
                          a.Hm1, a.Wm1);
    float gm = 0.0f, gdr = 0.0f, gdc = 0.0f;
    if (c.inside) {
      const bool vy0 = c.y0 >= 0, vy1 = c.y0 < a.H - 1;
      const bool vx0 = c.x0 >= 0, vx1 = c.x0 < a.W - 1;
      const bool ok[4] = {vy0 && vx0, vy0 && vx1, vy1 && vx0, vy1 && vx1};
      const float lh = c.lh, lw = c.lw, hh = 1.0f - lh, hw = 1.0f - lw;
      const float w[4] = {hh * hw, hh * lw, lh * hw, lh * lw};
      const int cy[4] = {c.y0, c.y0, c.y0 + 1, c.y0 + 1};
      const int cx[4] = {c.x0, c.x0 + 1, c.x0, c.x0 + 1};
      uint32_t q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        q[r] = ok[r] ? img_off + (uint32_t)(cy[r] * a.W + cx[r]) * pix_bytes : kOutside;
      float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // corner sums of gy * v
#pragma unroll 1
      for (int jv = (int)li; jv < b.nvec; jv += Lg) {
        u32x4 vv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vv[r] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(q[r] + 16u * (uint32_t)jv), 0, 0);
        const u32x4 gw = *reinterpret_cast<const u32x4*>(gyp + 16 * jv);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const float gyc = io::lane(gw, e);
#pragma unroll
          for (int r = 0; r < 4; ++r) S[r] = __builtin_fmaf(gyc, io::lane(vv[r], e), S[r]);
        }
      }
      point_grads(S, w, lh, lw, gm, gdr, gdc);
    }
    // the item's Lg lanes are consecutive and Lg-aligned in the wave
    for (int off = 1; off < Lg; off <<= 1) {
      gm += __shfl_xor(gm, off, 64);
      gdr += __shfl_xor(gdr, off, 64);
      gdc += __shfl_xor(gdc, off, 64);
    }
    if (li == 0) {
      float* row = om_rows + row0 * (uint32_t)(3 * K);
      const float mf = m * f;
      row[2 * k] = mf * gdc;      // dx moves the column
      row[2 * k + 1] = mf * gdr;  // dy moves the row
      row[2 * K + k] = gm;
    }
  }
  __syncthreads();
  // rows of this workgroup's items: one contiguous block from item0
  const int64_t item0 = ((int64_t)blockIdx.x * kBlock) >> b.lg_shift;
  const int64_t items_total = b.lanes >> b.lg_shift;
  const int64_t rows = min((int64_t)(kBlock >> b.lg_shift), items_total - item0);
  const int64_t vals = rows * (3 * K);
  float* go = b.gom + item0 * (3 * K);
  for (int64_t e = threadIdx.x; e < vals; e += kBlock) go[e] = om_rows[e];
}

// Tiled backward for the offset/weight gradients (grad_x gathered separately
// or not asked for): the forward's tile decomposition, LDS input window and
// staged offset/weight values; per point the same window test as the
// forward, the corners read from LDS (or, for a wave with a point outside the
// window, from global memory) and the three sums over the lane's channels
// kept in registers.  When a group spans L = 2 or 4 lanes their sums are
// added by xor-shuffles.  A group too wide for one window (channel slices:
// FlowDCN's 72 channels as three slices of 24) is done by one workgroup slice
// after slice, the window restaged for each and the sums added in slice
// order, so the result stays bit-reproducible.  Every mode (group scales:
// the lane's scale and the centre-based geometry of the forward).  3x3
// kernels.
struct BwdTileArgs {
  const char* gy;   // [N,Ho,Wo,C] I/O dtype, this launch
  float* gom;       // [N,Ho,Wo,G,3K] fp32, this launch (written)
  int32_t nslices;  // channel slices per group, done in turn (1: whole groups)
};

template <int DT, int VEC, int NV, int MODE, bool SL>
__global__ __launch_bounds__(kBlock) void dcn4_tile_bwd_kernel(TileArgs a, BwdTileArgs bb) {
  typedef Io<DT> io;
  constexpr int es = io::es;
  constexpr int DP = VEC * NV;
  constexpr int KS = 3, K = 9;
  extern __shared__ u32x4 lds_u4[];
  char* lds = reinterpret_cast<char*>(lds_u4);

  TileOrigin org = tile_origin(a);  // org.s: the slice in the window
  const uint32_t n = org.n, g0 = org.g0;
  const int ty0 = org.ty0, tx0 = org.tx0, wy0 = org.wy0, wx0 = org.wx0;
  const uint32_t t = threadIdx.x;
  const uint32_t pix_bytes = (uint32_t)(a.C * es);
  // 16-bit offset/weight rows, one group per workgroup: each lane reads its
  // row from global memory into registers (as the forward does), else the
  // rows are staged in LDS
  constexpr bool OMD_OK = es == 2;
  const bool omd = OMD_OK && a.om_direct != 0;
  uint32_t omw[kOmWords<es>];
  uint32_t mis;
  if (OMD_OK && omd) {
    mis = (g0 * (uint32_t)(27 * es)) & 3u;
    load_om_row<es>(a, n, g0, ty0, tx0, omw);
  } else {
    mis = stage_om<es>(a, org, K, lds + a.om_lds);
  }
  const rsrc_t xr = stage_window<es>(a, org, lds);
  __syncthreads();
  if (OMD_OK && omd && mis) {
    // the row starts at the odd 16-bit position: move it down by 16 bits so
    // that value j is half j of the words
#pragma unroll
    for (int q = 0; q + 1 < kOmWords<es>; ++q)
      omw[q] = __builtin_amdgcn_alignbit(omw[q + 1], omw[q], 16u);
    omw[kOmWords<es> - 1] >>= 16;
  }

  // ---- lane -> (tile pixel, group in chunk, channel slice)
  const uint32_t tp = fastdiv(t, a.div_gbl);
  const uint32_t rr = t - tp * (uint32_t)(a.GB * a.L);
  const uint32_t gl = fastdiv(rr, a.div_L), l = rr - gl * (uint32_t)a.L;
  const uint32_t py = fastdiv(tp, a.div_tw), px = tp - py * (uint32_t)a.TW;
  const int yo = ty0 + (int)py, xo = tx0 + (int)px;
  const bool active = yo < a.Ho && xo < a.Wo;
  const uint32_t g = g0 + gl;
  const typename io::raw* om = reinterpret_cast<const typename io::raw*>(
      lds + a.om_lds + tp * (uint32_t)(a.OSU * a.OMU) + mis + gl * (uint32_t)(3 * K * es));

  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  const uint32_t row_lds = (uint32_t)(a.WW * a.PS);
  const float row_f = (float)row_lds, ps_f = (float)a.PS;
  const float lane_f = (float)(lds_base + (gl * (uint32_t)a.D + l * DP) * es);
  const float ymax = (float)(a.WH - 2), xmax = (float)(a.WW - 2);
  constexpr bool GS = MODE == kGroupScale;
  constexpr int hy = (KS - 1) >> 1, hx = (KS - 1) >> 1;
  // point base: the grid point's row/column (standard), the centre (group scales)
  const int by0 = yo * a.sh - a.ph + (GS ? hy : 0), bx0 = xo * a.sw - a.pw + (GS ? hx : 0);
  const float ry0 = (float)(by0 - wy0), rx0 = (float)(bx0 - wx0);
  float sg = 1.0f;  // the lane's group scale (pixel 0 for idle lanes)
  if constexpr (GS) {
    FwdArgs fa{};
    fa.G = a.G; fa.scales = a.scales; fa.pscales = a.pscales; fa.max_scale = a.max_scale;
    sg = group_scale(fa, active ? ((uint64_t)n * a.Ho + (uint32_t)yo) * a.Wo + (uint32_t)xo : 0, g);
  }
  const float f = GS ? sg : (MODE == kStdScaled) ? a.offset_scale : 1.0f;
  // per point, summed over the slices: sum gy*dB/dcol, sum gy*dB/drow, sum gy*B
  float res[3 * K];  // then the lane's row of grad_offset_mask, in the tensor's order
#pragma unroll
  for (int c = 0; c < 3 * K; ++c) res[c] = 0.0f;

  const int nsl = SL ? bb.nslices : 1;
  for (int sl = 0; sl < nsl; ++sl) {
  if (SL && sl > 0) {
    __syncthreads();  // every wave is done with the previous slice's window
    org.s = (uint32_t)sl;
    stage_window<es>(a, org, lds);
    __syncthreads();
  }
  // first channel of the lane: group, slice, lane
  const uint32_t lane_bytes = (g * (uint32_t)a.D + (uint32_t)sl * (uint32_t)a.DSL + l * DP) * es;
  // upstream gradient of the lane's channels (pixel (0, 0) for idle lanes)
  float gyv[DP];
  {
    const char* gp = bb.gy + (((uint64_t)n * a.Ho + (active ? yo : 0)) * a.Wo + (active ? xo : 0)) *
                                 pix_bytes + lane_bytes;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(gp + 16 * v);
#pragma unroll
      for (int e = 0; e < VEC; ++e) gyv[v * VEC + e] = active ? io::lane(w, e) : 0.0f;
    }
  }

#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int i = k / KS, j = k - (k / KS) * KS;
    float dx, dy, m;
    if (OMD_OK && omd) {
      dx = om_packed<DT, 0>(omw, 2 * k);
      dy = om_packed<DT, 0>(omw, 2 * k + 1);
      m = om_packed<DT, 0>(omw, 2 * K + k);
    } else {
      dx = io::dec(om[2 * k]);
      dy = io::dec(om[2 * k + 1]);
      m = io::dec(om[2 * K + k]);
    }
    const float gyy = GS ? (float)(i - hy) : 0.0f, gxx = GS ? (float)(j - hx) : 0.0f;
    const Loc lc = sample_location<MODE>(GS ? ry0 : ry0 + (float)(i * a.dh),
                                         GS ? rx0 : rx0 + (float)(j * a.dw), gyy, gxx, dy, dx,
                                         a.offset_scale, sg);
    const float fy = __builtin_floorf(lc.ty), fx = __builtin_floorf(lc.tx);
    const float yr = lc.by + fy, xr_ = lc.bx + fx;  // corner (y0, x0), window-relative
    // whole-image window: a cell outside it is not inside the image, its
    // sample has zero gradient, and the lane reads window cell (0, 0)
    // instead; otherwise a cell outside the window sends the wave global
    const bool out = !(yr >= 0.0f) || !(yr <= ymax) || !(xr_ >= 0.0f) || !(xr_ <= xmax);
    const uint64_t off_window = a.whole ? 0 : __builtin_amdgcn_ballot_w64(active && out);
    float lh = 0.0f, lw = 0.0f;
    bool inside = true;
    u32x4 vv[4][NV];
    if (off_window == 0) {
      lh = lc.ty - fy;
      lw = lc.tx - fx;
      if (out) inside = false;  // whole-image window only
      const float yq = out ? 0.0f : yr, xq = out ? 0.0f : xr_;
      const uint32_t a00 = (uint32_t)__builtin_fmaf(yq, row_f, __builtin_fmaf(xq, ps_f, lane_f));
      LdsTap<DT, VEC, NV> d;
      d.load(a00, a00 + row_lds, a00 + 16u, a00 + row_lds + 16u, (uint32_t)a.PS);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int n2 = 0; n2 < NV; ++n2) vv[r][n2] = d.v[r][n2];
    } else {
      // global path: absolute location, global gathers (zero outside the image)
      const Cell cc = locate(sample_location<MODE>((float)(GS ? by0 : by0 + i * a.dh),
                                                   (float)(GS ? bx0 : bx0 + j * a.dw), gyy, gxx,
                                                   dy, dx, a.offset_scale, sg),
                             a.Hm1, a.Wm1);
      inside = cc.inside;
      lh = cc.lh;
      lw = cc.lw;
      const bool vy0 = cc.y0 >= 0, vy1 = cc.y0 < a.H - 1;
      const bool vx0 = cc.x0 >= 0, vx1 = cc.x0 < a.W - 1;
      const bool ok[4] = {inside && vy0 && vx0, inside && vy0 && vx1, inside && vy1 && vx0,
                          inside && vy1 && vx1};
      const int cy[4] = {cc.y0, cc.y0, cc.y0 + 1, cc.y0 + 1};
      const int cx[4] = {cc.x0, cc.x0 + 1, cc.x0, cc.x0 + 1};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t q = ok[r] ? lane_bytes + (uint32_t)(cy[r] * a.W + cx[r]) * pix_bytes : kOutside;
#pragma unroll
        for (int n2 = 0; n2 < NV; ++n2)
          vv[r][n2] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(q + 16 * n2), 0, 0);
      }
    }
    // a sample that is not inside reads only zeros: its sums stay zero
    const float hh = 1.0f - lh, hw = 1.0f - lw;
    const float w[4] = {hh * hw, hh * lw, lh * hw, lh * lw};
    float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // corner sums of gy * v
#pragma unroll
    for (int n2 = 0; n2 < NV; ++n2)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int c = n2 * VEC + e;
#pragma unroll
        for (int r = 0; r < 4; ++r) S[r] = __builtin_fmaf(gyv[c], io::lane(vv[r][n2], e), S[r]);
      }
    float gm, gdr, gdc;
    point_grads(S, w, lh, lw, gm, gdr, gdc);
    if (!inside) gm = gdr = gdc = 0.0f;
    // lanes of one (pixel, group) are consecutive; L is 1, 2 or 4
    for (int off = 1; off < a.L; off <<= 1) {
      gm += __shfl_xor(gm, off, 64);
      gdr += __shfl_xor(gdr, off, 64);
      gdc += __shfl_xor(gdc, off, 64);
    }
    if constexpr (SL) {
      res[2 * k] += gdc;      // dx moves the column
      res[2 * k + 1] += gdr;  // dy moves the row
      res[2 * K + k] += gm;
    } else {
      const float mf = m * f;
      res[2 * k] = mf * gdc;
      res[2 * k + 1] = mf * gdr;
      res[2 * K + k] = gm;
    }
  }
  }  // slices
  if constexpr (SL) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float mk = (OMD_OK && omd) ? om_packed<DT, 0>(omw, 2 * K + k) : io::dec(om[2 * K + k]);
      const float mf = mk * f;
      res[2 * k] = mf * res[2 * k];
      res[2 * k + 1] = mf * res[2 * k + 1];
    }
  }

  // Write-out through LDS: a row per (pixel, group) item, 3K floats at odd
  // stride (no bank conflicts), then each wave stores its own rows with
  // consecutive lanes on consecutive floats, so a store instruction touches
  // a few cache lines instead of one per lane.  The window and the staged
  // offsets are dead once every wave has finished its points.
  __syncthreads();
  const uint32_t l_shift = a.L == 4 ? 2u : a.L == 2 ? 1u : 0u;
  const uint32_t rows_wave = 64u >> l_shift;
  float* res_lds = reinterpret_cast<float*>(lds);
  uint64_t* base_lds = reinterpret_cast<uint64_t*>(lds + (uint32_t)(kBlock * 3 * K * 4) / (uint32_t)a.L);
  if (l == 0) {
    const uint32_t r = t >> l_shift;
#pragma unroll
    for (int c = 0; c < 3 * K; ++c) res_lds[r * (3 * K) + c] = res[c];
    base_lds[r] = active ? ((((uint64_t)n * a.Ho + yo) * a.Wo + xo) * (uint32_t)a.G + g) * (3 * K)
                         : ~uint64_t(0);
  }
  // each wave reads back only the rows its own lanes wrote, three floats (a
  // point's dx, dy gradients or three weight gradients) per lane and store
  typedef float f3 __attribute__((ext_vector_type(3), aligned(4)));
  const uint32_t wave = t >> 6, lane = t & 63u;
  const uint32_t r0 = wave * rows_wave;
  for (uint32_t e = lane; e < rows_wave * K; e += 64) {
    const uint32_t rl = e / K, c = 3 * (e - rl * K);
    const uint64_t base = base_lds[r0 + rl];
    if (base != ~uint64_t(0)) {
      const float* src = res_lds + (r0 + rl) * (3 * K) + c;
      const f3 v = {src[0], src[1], src[2]};
      *reinterpret_cast<f3*>(bb.gom + base + c) = v;
    }
  }
}

__global__ __launch_bounds__(kBlock) void dcn4_fill_zero_kernel(float* p, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t i = (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

// ------------------------------------------------------------ grad_x by gathering
// dL/dx is the adjoint of the bilinear gather: an inside sample (output pixel
// p, group g, point k) in the cell whose top-left corner is (y0, x0) adds
// fl(m*w_r) * dL/dy[p, c] to corner r of that cell, for each of the group's
// channels c.  As a scatter that is 4*D fp32 atomic lanes per sample; device
// atomics are served per 64-byte request (about 25e9 requests/s on this GPU,
// a request carrying the lanes of one instruction that fall in one 64-byte
// segment), so scattered atomics cost a request each.  Here the scatter
// becomes a gather:
//  1. bucket: a workgroup takes a tile of output pixels of one group and
//     counts its samples per cell in LDS (integer LDS atomics, which run at
//     full rate); one device atomic per non-empty cell of the tile's cell
//     window then reserves that cell's slots, and consecutive cells of a
//     window row are consecutive keys, so these coalesce; every sample
//     writes the record {p, m, lh, lw} (p = output row << xs | output
//     column) to its slot of the bucket of (image, group, cell), key =
//     row*(W+1) + x0+1 with row = (n*G + g)*(H+1) + y0+1.  Slot t of the buckets of one row is stored for all W+1 columns
//     side by side (record index (row*cap + t)*(W+1) + x0+1), so the gather's
//     lanes, which take consecutive columns, read consecutive records.  A
//     sample whose cell falls outside the window takes its slot with its own
//     device atomic.
//  2. gather: input pixel (y, x) is corner 00 of cell (y, x), 01 of
//     (y, x-1), 10 of (y-1, x) and 11 of (y-1, x-1).  A wave walks a strip
//     of bucket columns down a band of rows, reads each bucket's records
//     once and accumulates fl(m*w_r) * dL/dy per channel into one partial
//     sum per corner (fused multiply-add); a pixel adds the four partial
//     sums of its cells (one from the lane to its left, two from the
//     previous row) and is written once, so grad_x needs no clearing.
//  3. overflow: a bucket holds `cap` records; a sample whose slot is beyond
//     it is listed instead, and this launch adds its products with atomics
//     after the gather has written grad_x.
// The coefficients fl(m*w_r) are those of the atomic scatter; the order of
// each sum follows the slots, which depend on the order atomics were
// granted, so it varies from run to run as the scatter's does.
constexpr int kBucketNS = 8;  // samples per thread of a bucket workgroup

struct GatherArgs {
  FwdArgs f;           // geometry, om, scales, pscales of this chunk
  const char* gy;      // [imgs, Ho, Wo, C] I/O dtype
  float* gx;           // [imgs, H, W, C] fp32
  uint32_t* counts;    // [keys] records appended per bucket (may exceed cap)
  uint32_t* listed;    // [1] samples whose slot is beyond the capacity
  uint32_t* list;      // [samples] their ids
  u32x4* recs;         // [rows][cap][W+1] {p within its image, m, lh, lw} as bits
  uint32_t cap;
  uint32_t samples;    // samples of this chunk, < 2^31
  int32_t K, nchunk;  // nchunk: vectors of V channels per group
  int32_t Lg;         // gather: lanes per bucket column, min(nchunk, 16)
  int32_t nblocks;     // gather workgroups
  int32_t strips, bands;        // gather: column strips and row bands per (n, g)
  int32_t band_groups;          // gather workgroups per strip: kGatherWaves bands each
  int32_t band_rows;            // pixel rows of one band
  uint32_t xs;                  // bits of the output column in a record's pixel
  // gather: window of grad_y staged in LDS per workgroup (OWH x OWW output
  // pixels of the workgroup's group from (floor((y_lo + oy_off) / sh),
  // floor((cx0 + ox_off) / sw))); OWH = 0: not staged
  int32_t OWH, OWW, oy_off, ox_off;
  // bucket tiles: TH x TW output pixels (TW = 1 << tw_shift), their cell
  // window of WH x WW cells starting at (ty0*sh + wy_off, tx0*sw + wx_off)
  int32_t TH, tw_shift, WH, WW, wy_off, wx_off, tiles_x, tiles_y;
  // the chunk's groups: g0 .. g0 + gc - 1 (bucket keys, sample ids and
  // workgroups count groups from g0; tensors are addressed with g0 + local)
  int32_t g0, gc;
  FastDiv div_K, div_kw, div_gc, div_W, div_H, div_WW, div_tx, div_ty;
  FastDiv div_strips, div_bgroups, div_OWW, div_vpp;
};

struct SampleRec {
  uint32_t p;        // output pixel within its image, (yo << xs) | xo
  int y0, x0;
  float m, lh, lw;
  bool inside;
};

// The forward's sampling decisions (same device functions, same operation
// order) for point k of group g at output pixel (yo, xo); pix counts output
// pixels from the chunk's first image.
template <int DT, int MODE>
__device__ __forceinline__ SampleRec sample_at(const GatherArgs& ga, uint32_t pix, uint32_t yo,
                                               uint32_t xo, uint32_t g, int k) {
  typedef Io<DT> io;
  const FwdArgs& a = ga.f;
  const int i = (int)fastdiv((uint32_t)k, ga.div_kw), j = k - i * a.kw;
  const typename io::raw* om = reinterpret_cast<const typename io::raw*>(a.om) +
                               ((uint64_t)pix * (uint32_t)a.G + g) * (uint32_t)(3 * ga.K);
  const float dx = io::dec(om[2 * k]);
  const float dy = io::dec(om[2 * k + 1]);
  SampleRec r;
  r.m = io::dec(om[2 * ga.K + k]);
  float by, bx, gyy = 0.0f, gxx = 0.0f, sg = 1.0f;
  if (MODE == kGroupScale) {
    const int hy = (a.kh - 1) >> 1, hx = (a.kw - 1) >> 1;
    by = (float)((int)yo * a.sh - a.ph + hy);
    bx = (float)((int)xo * a.sw - a.pw + hx);
    gyy = (float)(i - hy);
    gxx = (float)(j - hx);
    sg = group_scale(a, pix, g);
  } else {
    by = (float)((int)yo * a.sh - a.ph + i * a.dh);
    bx = (float)((int)xo * a.sw - a.pw + j * a.dw);
  }
  const Cell c = locate(sample_location<MODE>(by, bx, gyy, gxx, dy, dx, a.offset_scale, sg),
                        a.Hm1, a.Wm1);
  r.p = (yo << ga.xs) | xo;
  r.y0 = c.y0;
  r.x0 = c.x0;
  r.lh = c.lh;
  r.lw = c.lw;
  r.inside = c.inside;
  return r;
}

__device__ __forceinline__ u32x4 pack_record(const SampleRec& r) {
  u32x4 rec;
  rec[0] = r.p;
  rec[1] = __float_as_uint(r.m);
  rec[2] = __float_as_uint(r.lh);
  rec[3] = __float_as_uint(r.lw);
  return rec;
}

// Bucket row of cell row y0 of the chunk's group gl in image n of the chunk;
// the cell (y0, x0) has key row*(W+1) + x0+1.
__device__ __forceinline__ uint64_t bucket_row(const GatherArgs& ga, uint32_t n, uint32_t gl,
                                               int y0) {
  return (uint64_t)(n * (uint32_t)ga.gc + gl) * (uint32_t)(ga.f.H + 1) + (uint32_t)(y0 + 1);
}

__device__ __forceinline__ void place_record(const GatherArgs& ga, uint64_t rowk, int x0,
                                             uint32_t slot, const u32x4& rec, uint32_t s) {
  if (slot < ga.cap) {
    const uint64_t cols = (uint32_t)(ga.f.W + 1);
    ga.recs[(rowk * ga.cap + slot) * cols + (uint32_t)(x0 + 1)] = rec;
  } else {
    const uint32_t at = atomicAdd(ga.listed, 1u);
    if (at < ga.samples) ga.list[at] = s;
  }
}

// Workgroup = (image n, group g, output tile); tile x fastest, then tile y,
// then g, then n.
template <int DT, int MODE>
__global__ __launch_bounds__(kBlock) void dcn4_bucket_kernel(GatherArgs ga) {
  extern __shared__ uint32_t cnt[];  // [WH*WW] counts, then reserved bases
  const FwdArgs& a = ga.f;
  uint32_t b = blockIdx.x;
  const uint32_t q1 = fastdiv(b, ga.div_tx);
  const uint32_t txi = b - q1 * (uint32_t)ga.tiles_x;
  const uint32_t q2 = fastdiv(q1, ga.div_ty);
  const uint32_t tyi = q1 - q2 * (uint32_t)ga.tiles_y;
  const uint32_t n = fastdiv(q2, ga.div_gc);
  const uint32_t gl = q2 - n * (uint32_t)ga.gc;  // group within the chunk
  const uint32_t g = (uint32_t)ga.g0 + gl;
  const int TW = 1 << ga.tw_shift;
  const int ty0 = (int)tyi * ga.TH, tx0 = (int)txi * TW;
  const int wy0 = ty0 * a.sh + ga.wy_off, wx0 = tx0 * a.sw + ga.wx_off;
  const int ncell = ga.WH * ga.WW;
  for (int i = threadIdx.x; i < ncell; i += kBlock) cnt[i] = 0;
  __syncthreads();
  const uint32_t nloc = (uint32_t)(ga.TH * TW * ga.K);
  const uint32_t img_pix = (uint32_t)(a.Ho * a.Wo);
  u32x4 rec[kBucketNS];
  int cell[kBucketNS];
  uint32_t rank[kBucketNS], sid[kBucketNS];
#pragma unroll
  for (int j = 0; j < kBucketNS; ++j) {
    cell[j] = -1;
    const uint32_t l = (uint32_t)j * kBlock + threadIdx.x;
    if (l >= nloc) continue;
    const uint32_t pl = fastdiv(l, ga.div_K);
    const int k = (int)(l - pl * (uint32_t)ga.K);
    const uint32_t yo = (uint32_t)ty0 + (pl >> ga.tw_shift);
    const uint32_t xo = (uint32_t)tx0 + (pl & (uint32_t)(TW - 1));
    if (yo >= (uint32_t)a.Ho || xo >= (uint32_t)a.Wo) continue;
    const uint32_t pix = n * img_pix + yo * (uint32_t)a.Wo + xo;
    const SampleRec r = sample_at<DT, MODE>(ga, pix, yo, xo, g, k);
    if (!r.inside) continue;
    rec[j] = pack_record(r);
    sid[j] = (pix * (uint32_t)ga.gc + gl) * (uint32_t)ga.K + (uint32_t)k;
    const int ly = r.y0 - wy0, lx = r.x0 - wx0;
    if ((unsigned)ly < (unsigned)ga.WH && (unsigned)lx < (unsigned)ga.WW) {
      cell[j] = ly * ga.WW + lx;
      rank[j] = atomicAdd(cnt + cell[j], 1u);
    } else {  // outside the window: a slot of its own
      const uint64_t rowk = bucket_row(ga, n, gl, r.y0);
      const uint32_t slot =
          atomicAdd(ga.counts + rowk * (uint32_t)(a.W + 1) + (uint32_t)(r.x0 + 1), 1u);
      place_record(ga, rowk, r.x0, slot, rec[j], sid[j]);
    }
  }
  __syncthreads();
  // one device atomic per non-empty cell reserves its slots
  for (int i = threadIdx.x; i < ncell; i += kBlock) {
    const uint32_t c = cnt[i];
    if (c == 0) continue;
    const int ly = (int)fastdiv((uint32_t)i, ga.div_WW), lx = i - ly * ga.WW;
    cnt[i] = atomicAdd(ga.counts + bucket_row(ga, n, gl, wy0 + ly) * (uint32_t)(a.W + 1) +
                           (uint32_t)(wx0 + lx + 1), c);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBucketNS; ++j) {
    if (cell[j] < 0) continue;
    const int ly = (int)fastdiv((uint32_t)cell[j], ga.div_WW), lx = cell[j] - ly * ga.WW;
    place_record(ga, bucket_row(ga, n, gl, wy0 + ly), wx0 + lx, cnt[cell[j]] + rank[j], rec[j],
                 sid[j]);
  }
}

// V consecutive elements widened to fp32 (one 16-byte load when they fill it).
template <int DT, int V>
__device__ __forceinline__ void load_widen(const typename Io<DT>::raw* p, float* v) {
  typedef Io<DT> io;
  if constexpr (V * io::es == 16) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = io::lane(q, e);
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) v[e] = io::dec(p[e]);
  }
}


// Waves per gather workgroup: consecutive bands of one strip.
constexpr int kGatherWaves = 4;

__device__ __forceinline__ int floor_div(int a, int b) {
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

// A wave owns (image n, group g, band of pixel rows [y_lo, y_hi), strip of
// Lc = floor(64 / Lg) bucket columns [cx0, cx0 + Lc)); lane (lc, li) =
// (lane / Lg, lane % Lg) takes bucket column cx0 + lc and the group's
// channel vectors li, li + Lg, ...  Lg is the group's vector count (at most
// 16), not rounded to a power of two, so a group of 9 vectors keeps 63 of
// the 64 lanes busy; lanes past the last column only idle.
// It walks bucket rows cy = y_lo .. y_hi; each bucket's records are read once
// and summed into four partial sums, one per corner of the cell:
//   S_r[c] = sum over the bucket's records of fl(m*w_r) * dL/dy[p, c].
// Bucket (cy, cx) holds the cell (cy-1, cx-1), so pixel (cy-1, cx-1) is
// complete after row cy:
//   (S_00(cy, cx) + S_10(cy-1, cx)) + (S_01(cy, cx-1) + S_11(cy-1, cx-1)),
// the cx-1 terms from the lane Lg to the left (one shuffle), the cy-1 terms
// kept from the previous row.  Strips overlap by one column; the strip's
// first lane only feeds its right neighbour, and the band's first row only
// the next row.
// A workgroup is kGatherWaves bands of one strip.  STAGE: it first copies
// the grad_y vectors of its group at the output pixels its cells' samples
// come from when their displacement is within the margin (a window of
// OWH x OWW pixels) to LDS; a record from outside the window reads grad_y
// from global memory.  Each vector is then fetched from global memory once
// per workgroup instead of once per record (K records per output pixel).
// U: records taken per round of a lane's bucket loop; their loads, then
// their grad_y loads, are all in flight before the first is used.
template <int DT, int V, bool VST, bool STAGE, int U>
__global__ __launch_bounds__(kBlock) void dcn4_gather_kernel(GatherArgs ga) {
  typedef Io<DT> io;
  constexpr int es = io::es;
  extern __shared__ u32x4 gather_lds[];
  const FwdArgs& a = ga.f;
  const uint32_t wg = (uint32_t)xcd_block(blockIdx.x, ga.nblocks);
  const uint32_t q1 = fastdiv(wg, ga.div_strips);
  const uint32_t strip = wg - q1 * (uint32_t)ga.strips;
  const uint32_t q2 = fastdiv(q1, ga.div_bgroups);
  const uint32_t bgrp = q1 - q2 * (uint32_t)ga.band_groups;
  const uint32_t n = fastdiv(q2, ga.div_gc);
  const uint32_t gl = q2 - n * (uint32_t)ga.gc;  // group within the chunk
  const uint32_t g = (uint32_t)ga.g0 + gl;
  const int lane = (int)(threadIdx.x & 63);
  const int wave = (int)(threadIdx.x >> 6);
  const int Lg = ga.Lg;
  const int lc = lane / Lg, li = lane - lc * Lg;
  const int Lc = 64 / Lg;
  const int cx0 = (int)strip * (Lc - 1);
  const int wy_lo = (int)bgrp * (kGatherWaves * ga.band_rows);
  const typename io::raw* gyn = reinterpret_cast<const typename io::raw*>(ga.gy) +
                                (uint64_t)n * (uint32_t)(a.Ho * a.Wo) * (uint32_t)a.C +
                                g * (uint32_t)a.D;
  const uint32_t pbytes = (uint32_t)(a.D * es);  // bytes of one staged pixel
  int oy0 = 0, ox0 = 0;
  if constexpr (STAGE) {
    oy0 = floor_div(wy_lo + ga.oy_off, a.sh);
    ox0 = floor_div(cx0 + ga.ox_off, a.sw);
    const uint32_t vpp = pbytes >> 4;  // 16-byte vectors per pixel
    const uint32_t total = (uint32_t)(ga.OWH * ga.OWW) * vpp;
    char* lds = reinterpret_cast<char*>(gather_lds);
    for (uint32_t i = threadIdx.x; i < total; i += kBlock) {
      const uint32_t pix = fastdiv(i, ga.div_vpp), v = i - pix * vpp;
      const uint32_t wy = fastdiv(pix, ga.div_OWW), wx = pix - wy * (uint32_t)ga.OWW;
      const int yo = oy0 + (int)wy, xo = ox0 + (int)wx;
      if ((unsigned)yo < (unsigned)a.Ho && (unsigned)xo < (unsigned)a.Wo)
        *reinterpret_cast<u32x4*>(lds + pix * pbytes + v * 16u) = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(gyn + ((uint32_t)yo * (uint32_t)a.Wo + (uint32_t)xo) *
                                                    (uint32_t)a.C) + v * 16u);
    }
    __syncthreads();  // the only barrier: waves without a band may leave after it
  }
  const int band = (int)bgrp * kGatherWaves + wave;
  if (band >= ga.bands) return;
  const int cx = cx0 + lc;
  const bool col_ok = lc < Lc && cx <= a.W;
  const int y_lo = band * ga.band_rows;
  const int y_hi = min(y_lo + ga.band_rows, a.H);
  const uint64_t row = (uint32_t)(a.W + 1);
  const uint64_t rk0 = (uint64_t)(n * (uint32_t)ga.gc + gl) * (uint32_t)(a.H + 1);  // bucket row 0
  const uint64_t kb = rk0 * row + (uint32_t)(col_ok ? cx : 0);
  float* gxn = ga.gx + (uint64_t)n * (uint32_t)(a.H * a.W) * (uint32_t)a.C + g * (uint32_t)a.D;
  const uint32_t xmask = (1u << ga.xs) - 1u;
  const int rounds = (ga.nchunk + Lg - 1) / Lg;
  for (int rd = 0; rd < rounds; ++rd) {
    const int jc = li + rd * Lg;
    const bool ch_ok = jc < ga.nchunk;
    const bool live = col_ok && ch_ok;
    float p10[V], p11[V];
#pragma unroll
    for (int e = 0; e < V; ++e) p10[e] = p11[e] = 0.0f;
    uint32_t cnt_next = live ? min(ga.counts[kb + (uint64_t)y_lo * row], ga.cap) : 0u;
#pragma unroll 1
    for (int cy = y_lo; cy <= y_hi; ++cy) {
      const uint32_t cnt = cnt_next;
      const uint64_t key = kb + (uint64_t)cy * row;
      if (cy < y_hi) cnt_next = live ? min(ga.counts[key + row], ga.cap) : 0u;
      float s00[V], s01[V], s10[V], s11[V];
#pragma unroll
      for (int e = 0; e < V; ++e) s00[e] = s01[e] = s10[e] = s11[e] = 0.0f;
      // slot t of this bucket: rp[t * row]
      const u32x4* rp = ga.recs + ((rk0 + (uint32_t)cy) * ga.cap) * row + (uint32_t)(col_ok ? cx : 0);
#pragma unroll 1
      for (uint32_t t0 = 0; t0 < cnt; t0 += U) {
        u32x4 rc[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (t0 + u < cnt) rc[u] = rp[(uint64_t)(t0 + u) * row];
        float v[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (t0 + u >= cnt) continue;
          const uint32_t yo = rc[u][0] >> ga.xs, xo = rc[u][0] & xmask;
          bool staged = false;
          if constexpr (STAGE) {
            const uint32_t wy = yo - (uint32_t)oy0, wx = xo - (uint32_t)ox0;
            staged = wy < (uint32_t)ga.OWH && wx < (uint32_t)ga.OWW;
            if (staged) {
              const char* lds = reinterpret_cast<const char*>(gather_lds);
              const u32x4 q = *reinterpret_cast<const u32x4*>(
                  lds + (wy * (uint32_t)ga.OWW + wx) * pbytes + (uint32_t)(jc * V * es));
#pragma unroll
              for (int e = 0; e < V; ++e) v[u][e] = io::lane(q, e);
            }
          }
          if (!staged)
            load_widen<DT, V>(gyn + (yo * (uint32_t)a.Wo + xo) * (uint32_t)a.C + jc * V, v[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (t0 + u >= cnt) break;
          const float m = __uint_as_float(rc[u][1]);
          const float lh = __uint_as_float(rc[u][2]), lw = __uint_as_float(rc[u][3]);
          const float hh = 1.0f - lh, hw = 1.0f - lw;
          const float c00 = m * (hh * hw), c01 = m * (hh * lw);
          const float c10 = m * (lh * hw), c11 = m * (lh * lw);
#pragma unroll
          for (int e = 0; e < V; ++e) {
            s00[e] = __builtin_fmaf(c00, v[u][e], s00[e]);
            s01[e] = __builtin_fmaf(c01, v[u][e], s01[e]);
            s10[e] = __builtin_fmaf(c10, v[u][e], s10[e]);
            s11[e] = __builtin_fmaf(c11, v[u][e], s11[e]);
          }
        }
      }
      if (cy > y_lo) {  // pixel row cy - 1 is complete
        float left[V];
#pragma unroll
        for (int e = 0; e < V; ++e) left[e] = __shfl_up(s01[e] + p11[e], (unsigned)Lg, 64);
        if (live && lc > 0) {
          float* o = gxn + ((uint64_t)(cy - 1) * (uint32_t)a.W + (uint32_t)(cx - 1)) *
                               (uint32_t)a.C + jc * V;
          float r[V];
#pragma unroll
          for (int e = 0; e < V; ++e) r[e] = (s00[e] + p10[e]) + left[e];
          if constexpr (VST && V % 4 == 0) {
#pragma unroll
            for (int e = 0; e < V; e += 4)
              *reinterpret_cast<float4*>(o + e) = make_float4(r[e], r[e + 1], r[e + 2], r[e + 3]);
          } else {
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = r[e];
          }
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        p10[e] = s10[e];
        p11[e] = s11[e];
      }
    }
  }
}

// Sample s = ((pix*G) + g)*K + k of the chunk.
template <int DT, int MODE>
__device__ __forceinline__ SampleRec sample_record(const GatherArgs& ga, uint32_t s,
                                                   uint32_t* n_out, uint32_t* g_out) {
  const FwdArgs& a = ga.f;
  const uint32_t item = fastdiv(s, ga.div_K);
  const int k = (int)(s - item * (uint32_t)ga.K);
  const uint32_t pix = fastdiv(item, ga.div_gc);
  const uint32_t g = (uint32_t)ga.g0 + (item - pix * (uint32_t)ga.gc);
  const uint32_t n = fastdiv(pix, a.div_hw);
  const uint32_t rem = pix - n * (uint32_t)(a.Ho * a.Wo);
  const uint32_t yo = fastdiv(rem, a.div_wo);
  const uint32_t xo = rem - yo * (uint32_t)a.Wo;
  *n_out = n;
  *g_out = g;
  return sample_at<DT, MODE>(ga, pix, yo, xo, g, k);
}

template <int DT, int MODE>
__device__ __forceinline__ void overflow_sample(const GatherArgs& ga, uint32_t s, uint32_t c) {
  typedef Io<DT> io;
  const FwdArgs& a = ga.f;
  uint32_t n, g;
  const SampleRec r = sample_record<DT, MODE>(ga, s, &n, &g);  // listed samples are inside
  const float gyc = io::dec(reinterpret_cast<const typename io::raw*>(ga.gy)[
      ((uint64_t)n * (uint32_t)(a.Ho * a.Wo) + (r.p >> ga.xs) * (uint32_t)a.Wo +
       (r.p & ((1u << ga.xs) - 1u))) * (uint32_t)a.C + g * (uint32_t)a.D + c]);
  const float hh = 1.0f - r.lh, hw = 1.0f - r.lw;
  const float w[4] = {hh * hw, hh * r.lw, r.lh * hw, r.lh * r.lw};
  const bool vy0 = r.y0 >= 0, vy1 = r.y0 < a.H - 1, vx0 = r.x0 >= 0, vx1 = r.x0 < a.W - 1;
  const bool ok[4] = {vy0 && vx0, vy0 && vx1, vy1 && vx0, vy1 && vx1};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!ok[q]) continue;
    const uint32_t cy = (uint32_t)(r.y0 + (q >> 1)), cx = (uint32_t)(r.x0 + (q & 1));
    unsafeAtomicAdd(ga.gx + ((uint64_t)(n * (uint32_t)a.H + cy) * (uint32_t)a.W + cx) *
                                (uint32_t)a.C + g * (uint32_t)a.D + c,
                    (r.m * w[q]) * gyc);
  }
}

// Grid-stride over (listed sample, channel); exits at once when none is listed.
template <int DT>
__global__ __launch_bounds__(kBlock) void dcn4_overflow_kernel(GatherArgs ga, int32_t mode) {
  const uint32_t listed = min(*ga.listed, ga.samples);
  const uint32_t D = (uint32_t)ga.f.D;
  const uint64_t total = (uint64_t)listed * D;
  const uint64_t stride = (uint64_t)gridDim.x * kBlock;
  for (uint64_t t = (uint64_t)blockIdx.x * kBlock + threadIdx.x; t < total; t += stride) {
    const uint32_t e = (uint32_t)(t / D);
    const uint32_t c = (uint32_t)(t - (uint64_t)e * D);
    const uint32_t s = ga.list[e];
    if (mode == kStdUnitScale) overflow_sample<DT, kStdUnitScale>(ga, s, c);
    else if (mode == kStdScaled) overflow_sample<DT, kStdScaled>(ga, s, c);
    else overflow_sample<DT, kGroupScale>(ga, s, c);
  }
}

// ------------------------------------------------------------ geometry probe
// One thread per (pixel, g, k); reads the merged tensor straight from global
// memory and writes what the forward kernel's geometry functions compute.
template <int DT, int MODE>
__global__ __launch_bounds__(kBlock) void dcn4_probe_kernel(
    FwdArgs a, int32_t* y0, int32_t* x0, float* lh, float* lw,
    uint8_t* inside, int64_t count) {
  typedef Io<DT> io;
  const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= count) return;
  const int K = a.kh * a.kw;
  const int64_t pg = t / K;
  const int k = (int)(t - pg * K);
  const int64_t p = pg / a.G;
  const int g = (int)(pg - p * a.G);
  const int64_t hw = (int64_t)a.Ho * a.Wo;
  const int rem = (int)(p % hw);
  const int yo = rem / a.Wo, xo = rem % a.Wo;
  const int i = k / a.kw, j = k % a.kw;
  const typename io::raw* om =
      reinterpret_cast<const typename io::raw*>(a.om) + (p * a.G + g) * (3 * K);
  const float dx = io::dec(om[2 * k]);
  const float dy = io::dec(om[2 * k + 1]);
  const float sg = (MODE == kGroupScale) ? group_scale(a, (uint64_t)p, (uint32_t)g) : 1.0f;
  const int hy = (a.kh - 1) >> 1, hx = (a.kw - 1) >> 1;
  float by, bx, gy = 0.0f, gx = 0.0f;
  if (MODE == kGroupScale) {
    by = (float)(yo * a.sh - a.ph + hy);
    bx = (float)(xo * a.sw - a.pw + hx);
    gy = (float)(i - hy);
    gx = (float)(j - hx);
  } else {
    by = (float)(yo * a.sh - a.ph + i * a.dh);
    bx = (float)(xo * a.sw - a.pw + j * a.dw);
  }
  const Cell c = locate(sample_location<MODE>(by, bx, gy, gx, dy, dx,
                                              a.offset_scale, sg),
                        a.Hm1, a.Wm1);
  inside[t] = c.inside ? 1 : 0;
  y0[t] = c.inside ? c.y0 : 0;
  x0[t] = c.inside ? c.x0 : 0;
  lh[t] = c.inside ? c.lh : 0.0f;
  lw[t] = c.inside ? c.lw : 0.0f;
}

// ------------------------------------------------------------ host launchers
#ifndef DCN4_TILE_PART_DT
typedef void (*fwd_fn)(FwdArgs);

template <int DT, int VEC, int NV, int MODE>
fwd_fn pick_ks(int K3) {
  return K3 ? dcn4_forward_kernel<DT, VEC, NV, MODE, 3>
            : dcn4_forward_kernel<DT, VEC, NV, MODE, 0>;
}

template <int DT, int VEC, int NV>
fwd_fn pick_mode(int mode, int K3) {
  switch (mode) {
    case kStdUnitScale: return pick_ks<DT, VEC, NV, kStdUnitScale>(K3);
    case kStdScaled: return pick_ks<DT, VEC, NV, kStdScaled>(K3);
    default: return pick_ks<DT, VEC, NV, kGroupScale>(K3);
  }
}

template <int DT>
fwd_fn pick_vec(bool vector_path, int nv, int mode, int K3) {
  constexpr int V = 16 / Io<DT>::es;
  if (!vector_path) return pick_mode<DT, 1, 1>(mode, K3);
  switch (nv) {
    case 1: return pick_mode<DT, V, 1>(mode, K3);
    case 2: return pick_mode<DT, V, 2>(mode, K3);
    case 3: return pick_mode<DT, V, 3>(mode, K3);
    default: return pick_mode<DT, V, 4>(mode, K3);
  }
}

fwd_fn pick_forward(int dtype, bool vector_path, int nv, int mode, int K3) {
  switch (dtype) {
    case DCN4_F32: return pick_vec<DCN4_F32>(vector_path, nv, mode, K3);
    case DCN4_BF16: return pick_vec<DCN4_BF16>(vector_path, nv, mode, K3);
    default: return pick_vec<DCN4_F16>(vector_path, nv, mode, K3);
  }
}

void fill_common(const Plan& p, FwdArgs& a) {
  const dcn4_desc& d = p.desc;
  a.H = d.H; a.W = d.W; a.C = d.C; a.G = d.group; a.D = p.D;
  a.Ho = p.Ho; a.Wo = p.Wo;
  a.kh = d.kernel_h; a.kw = d.kernel_w; a.sh = d.stride_h; a.sw = d.stride_w;
  a.ph = d.pad_h; a.pw = d.pad_w; a.dh = d.dilation_h; a.dw = d.dilation_w;
  a.offset_scale = d.offset_scale;
  a.max_scale = d.use_group_scales ? d.max_scale : 0.0f;
  a.Hm1 = (float)(d.H - 1);
  a.Wm1 = (float)(d.W - 1);
  a.rowel = d.group * 3 * p.K;
  a.img_bytes = (uint32_t)((uint64_t)d.H * d.W * d.C * p.es);
  a.div_hw = make_fastdiv((uint32_t)(p.Ho * p.Wo));
  a.div_wo = make_fastdiv((uint32_t)p.Wo);
}


#endif  // !DCN4_TILE_PART_DT

template <int DT, int NV, int MODE, bool WHOLE>
tile_fn tile_kw(int K3, bool psc) {
  constexpr int V = 16 / Io<DT>::es;
  if (!K3) return dcn4_tile_kernel<DT, V, NV, MODE, 0, 0, WHOLE>;
  return psc ? dcn4_tile_kernel<DT, V, NV, MODE, 3, 16 * NV, WHOLE>
             : dcn4_tile_kernel<DT, V, NV, MODE, 3, 0, WHOLE>;
}

// whole: the whole-image window, an instantiation of its own so that the
// margin window's point loop carries no test of the window kind
template <int DT, int NV, int MODE>
tile_fn tile_ks(int K3, bool psc, bool whole) {
  return whole ? tile_kw<DT, NV, MODE, true>(K3, psc) : tile_kw<DT, NV, MODE, false>(K3, psc);
}

template <int DT, int MODE>
tile_fn tile_pick_nv(int nv, int K3, bool psc, bool whole) {
  switch (nv) {
    case 1: return tile_ks<DT, 1, MODE>(K3, psc, whole);
    case 2: return tile_ks<DT, 2, MODE>(K3, psc, whole);
    case 3: return tile_ks<DT, 3, MODE>(K3, psc, whole);
    default: return tile_ks<DT, 4, MODE>(K3, psc, whole);
  }
}

}  // namespace

#ifdef DCN4_TILE_PART_DT
// A translation unit of its own per (dtype, mode) pair instantiates that
// pair's tiled forward kernels (dcn4_tile_part.hip), so the library's
// kernels compile in parallel.
tile_fn DCN4_TILE_PART_FN(DCN4_TILE_PART_DT, DCN4_TILE_PART_MODE)(int nv, int K3, bool psc,
                                                                  bool whole) {
  return tile_pick_nv<DCN4_TILE_PART_DT, DCN4_TILE_PART_MODE>(nv, K3, psc, whole);
}
}  // namespace dcn4
#else
namespace {

tile_fn tile_pick(int dtype, int mode, int nv, int K3, bool psc, bool whole) {
#define DCN4_TILE_CASE(DT, MODE) \
  if (dtype == DT && mode == MODE) return DCN4_TILE_PART_FN(DT, MODE)(nv, K3, psc, whole);
  DCN4_TILE_CASE(0, 0) DCN4_TILE_CASE(0, 1) DCN4_TILE_CASE(0, 2)
  DCN4_TILE_CASE(1, 0) DCN4_TILE_CASE(1, 1) DCN4_TILE_CASE(1, 2)
  DCN4_TILE_CASE(2, 0) DCN4_TILE_CASE(2, 1) DCN4_TILE_CASE(2, 2)
#undef DCN4_TILE_CASE
  return nullptr;
}

}  // namespace

thread_local char g_hip_error[128] = "";

void note_hip_error(hipError_t e) {
  snprintf(g_hip_error, sizeof g_hip_error, "%s (%d): %s", hipGetErrorName(e),
           (int)e, hipGetErrorString(e));
}

const char* last_hip_error() { return g_hip_error; }

int32_t forward_lds_bytes(const Plan& p, int32_t lanes_per_group, int32_t block) {
  // pixels a range of `block` items can touch, plus one 16-byte alignment lead
  const int64_t ipp = (int64_t)p.desc.group * lanes_per_group;
  const int64_t pixels = (block + ipp - 1) / ipp + 1;
  const int64_t bytes = pixels * p.desc.group * 3 * p.K * p.es + 16;
  return (int32_t)((bytes + 15) & ~int64_t(15));
}

int32_t forward_block(const Plan& p, int32_t lanes_per_group) {
  for (int32_t b = kBlock; b >= 64; b >>= 1)
    if (forward_lds_bytes(p, lanes_per_group, b) <= kLdsBudget) return b;
  return 0;
}

dcn4_status launch_forward(const Plan& p, const void* x, const void* om,
                           const float* scales, const float* pscales, void* y,
                           void* stream, bool vector_path) {
  const dcn4_desc& d = p.desc;
  const int dp = vector_path ? p.dp : 1;
  const int L = p.D / dp;
  const int K3 = (d.kernel_h == 3 && d.kernel_w == 3) ? 1 : 0;
  fwd_fn fn = pick_forward(d.dtype, vector_path, dp / (16 / p.es), p.mode, K3);
  const int32_t block = forward_block(p, L);
  if (block == 0) return DCN4_ERR_UNSUPPORTED;
  const int32_t lds = forward_lds_bytes(p, L, block);
  FwdArgs a{};
  fill_common(p, a);
  a.scales = scales;
  a.L = L;
  const uint64_t ps_img = (uint64_t)p.Ho * p.Wo * d.group;  // pixel scales per image
  a.ipp = d.group * L;
  a.div_ipp = make_fastdiv((uint32_t)a.ipp);
  a.div_L = make_fastdiv((uint32_t)L);
  const uint64_t x_img = (uint64_t)d.H * d.W * d.C * p.es;
  const uint64_t y_img = (uint64_t)p.Ho * p.Wo * d.C * p.es;
  const uint64_t om_img = (uint64_t)p.Ho * p.Wo * a.rowel * p.es;
  for (int32_t n0 = 0; n0 < d.N; n0 += p.images_per_launch) {
    const int32_t nb = (d.N - n0) < p.images_per_launch ? (d.N - n0) : p.images_per_launch;
    a.x = static_cast<const char*>(x) + n0 * x_img;
    a.om = static_cast<const char*>(om) + n0 * om_img;
    a.y = static_cast<char*>(y) + n0 * y_img;
    a.pscales = pscales ? pscales + n0 * ps_img : nullptr;
    a.x_bytes = nb * x_img;
    a.om_bytes = nb * om_img;
    a.total_items = (int32_t)((int64_t)nb * p.Ho * p.Wo * a.ipp);
    a.block = block;
    a.nblocks = (a.total_items + block - 1) / block;
    hipLaunchKernelGGL(fn, dim3(a.nblocks), dim3(block), lds,
                       static_cast<hipStream_t>(stream), a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      note_hip_error(e);
      return DCN4_ERR_HIP;
    }
  }
  return DCN4_OK;
}

dcn4_status launch_dcnv3_softmax(const Plan& p, const void* om, void* out, void* stream) {
  const dcn4_desc& d = p.desc;
  const uint64_t rows = (uint64_t)d.N * p.Ho * p.Wo * d.group;
  const int32_t row_bytes = 3 * p.K * p.es;
  int32_t R = kDcnv3SoftmaxLds / row_bytes;
  if (R > kBlock) R = kBlock;
  if (R < 1) return DCN4_ERR_UNSUPPORTED;
  const uint64_t nb = (rows + R - 1) / R;
  if (nb > 0x7fffffffu) return DCN4_ERR_UNSUPPORTED;
  const int32_t lds = R * row_bytes;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (d.dtype) {
    case DCN4_F32:
      hipLaunchKernelGGL(dcn4_dcnv3_softmax_kernel<DCN4_F32>, dim3((uint32_t)nb), dim3(kBlock), lds, st,
                         static_cast<const float*>(om), static_cast<float*>(out), rows, p.K, R);
      break;
    case DCN4_BF16:
      hipLaunchKernelGGL(dcn4_dcnv3_softmax_kernel<DCN4_BF16>, dim3((uint32_t)nb), dim3(kBlock), lds, st,
                         static_cast<const uint16_t*>(om), static_cast<uint16_t*>(out), rows, p.K, R);
      break;
    default:
      hipLaunchKernelGGL(dcn4_dcnv3_softmax_kernel<DCN4_F16>, dim3((uint32_t)nb), dim3(kBlock), lds, st,
                         static_cast<const uint16_t*>(om), static_cast<uint16_t*>(out), rows, p.K, R);
      break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    note_hip_error(e);
    return DCN4_ERR_HIP;
  }
  return DCN4_OK;
}

template <int DT>
fwd_fn dcnv3_pick(int mode, int K3) {
  if (mode == kStdUnitScale)
    return K3 ? dcn4_dcnv3_kernel<DT, kStdUnitScale, 3> : dcn4_dcnv3_kernel<DT, kStdUnitScale, 0>;
  return K3 ? dcn4_dcnv3_kernel<DT, kStdScaled, 3> : dcn4_dcnv3_kernel<DT, kStdScaled, 0>;
}

dcn4_status launch_dcnv3(const Plan& p, const void* x, const void* om, void* y, void* stream) {
  const dcn4_desc& d = p.desc;
  if (p.mode == kGroupScale) return DCN4_ERR_UNSUPPORTED;
  const int K3 = (d.kernel_h == 3 && d.kernel_w == 3) ? 1 : 0;
  fwd_fn fn = d.dtype == DCN4_F32 ? dcnv3_pick<DCN4_F32>(p.mode, K3)
            : d.dtype == DCN4_BF16 ? dcnv3_pick<DCN4_BF16>(p.mode, K3)
                                   : dcnv3_pick<DCN4_F16>(p.mode, K3);
  FwdArgs a{};
  fill_common(p, a);
  a.L = p.D;
  a.ipp = d.C;
  a.div_ipp = make_fastdiv((uint32_t)d.C);
  a.div_L = make_fastdiv((uint32_t)p.D);
  const uint64_t x_img = (uint64_t)d.H * d.W * d.C * p.es;
  const uint64_t y_img = (uint64_t)p.Ho * p.Wo * d.C * p.es;
  const uint64_t om_img = (uint64_t)p.Ho * p.Wo * a.rowel * p.es;
  for (int32_t n0 = 0; n0 < d.N; n0 += p.images_per_launch) {
    const int32_t nb = (d.N - n0) < p.images_per_launch ? (d.N - n0) : p.images_per_launch;
    a.x = static_cast<const char*>(x) + n0 * x_img;
    a.om = static_cast<const char*>(om) + n0 * om_img;
    a.y = static_cast<char*>(y) + n0 * y_img;
    a.x_bytes = nb * x_img;
    a.om_bytes = nb * om_img;
    a.total_items = (int32_t)((int64_t)nb * p.Ho * p.Wo * d.C);
    a.block = kBlock;
    a.nblocks = (a.total_items + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(fn, dim3(a.nblocks), dim3(kBlock), 0, static_cast<hipStream_t>(stream), a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      note_hip_error(e);
      return DCN4_ERR_HIP;
    }
  }
  return DCN4_OK;
}

namespace {

// Tile shape for `gb` groups per workgroup and `dp` channels per lane;
// false when it does not fit (lanes, staging passes or LDS).
// slices > 1: chunks of one group's dp channels (one lane per pixel, the
// window holds the slice only); slices == 1: chunks of gb whole groups.
// Tile height and width for tp tile pixels (a power of two up to 256).
void tile_dims(int32_t tp, int32_t& th, int32_t& tw) {
  tw = tp >= 16 ? 16 : tp;
  th = tp / tw;
  if (tp == 64) { th = 8; tw = 8; }
}

bool tile_shape_mp(const Plan& p, int32_t dp, int32_t gb, int32_t slices, bool whole,
                   int32_t mp, TileShape& t) {
  const dcn4_desc& d = p.desc;
  if (slices < 1 || (slices > 1 && (gb != 1 || dp * slices != p.D))) return false;
  const int32_t L = slices > 1 ? 1 : p.D / dp;
  const int32_t lanes_px = gb * L;
  if (gb < 1 || d.group % gb || lanes_px > kBlock || kBlock % lanes_px) return false;
  const int32_t tp = kBlock / lanes_px;  // tile pixels
  int32_t th, tw;
  tile_dims(tp, th, tw);
  const int32_t M = p.tile_margin;
  // margin window: mp consecutive tile rows per workgroup under one staging
  if (whole) mp = 1;
  // the footprint of the tile rows' points plus the margin (and one more for
  // the bilinear corners), or the image with a zero row/column on every side
  const int32_t wh = whole ? d.H + 2
                           : (th * mp - 1) * d.stride_h + (d.kernel_h - 1) * d.dilation_h + 2 * M + 2;
  const int32_t ww = whole ? d.W + 2
                           : (tw - 1) * d.stride_w + (d.kernel_w - 1) * d.dilation_w + 2 * M + 2;
  const int32_t cb = slices > 1 ? dp * p.es : gb * p.D * p.es;
  if (cb % 16) return false;
  int32_t ps = cb;
  if (p.tile_pad && ((ps / 16) % 2 == 0)) ps += 16;  // odd number of 16-byte chunks
  if ((int64_t)ww * (ps / 16) > kBlock) return false;  // a window row per pass
  // offset/weight units: the chunk's values from the 4-byte boundary below
  // their start (a 2-byte lead when 16-bit values start mid-word), in units
  // of 4 or 16 bytes
  const int32_t ob = gb * 3 * p.K * p.es + (p.es == 2 ? 2 : 0);
  const int64_t win = (int64_t)wh * ww * ps;
  // window, offset/weight values, and (bf16) 16 bytes for the workgroup's
  // agreement on the window encoding
  auto lds_for = [&](int32_t u) {
    const int32_t n = (ob + u - 1) / u;
    return ((win + 15) & ~int64_t(15)) + (int64_t)tp * n * u + (d.dtype == DCN4_BF16 ? 16 : 0);
  };
  const int64_t lds4 = lds_for(4);
  if ((ob + 3) / 4 > kBlock || lds4 > 64 * 1024) return false;
  // automatic unit: 16 bytes (a quarter of the copy instructions) when that
  // keeps the workgroups per CU and the lanes' reads of their values stay at
  // most 4-way bank conflicted: a lane reads its pixel's values at a stride
  // of osu * 16 bytes, so 64 lanes share gcd(osu * 4, 64) of the 64 banks'
  // 4-byte words per bank (measured: 16-byte units on the 56-byte bf16 rows
  // of the U-Net block, a 64-byte stride, 120.6 -> 134.0 us; on the fp32
  // InternImage stage, a 112-byte stride, 68.1 -> 61.2 us)
  int32_t omu = 4;
  if (p.tile_om_unit == 1) {
    omu = 4;  // the backward's staging (and the forward's where rows cannot be read directly)
  } else if (p.tile_om_unit) {
    omu = p.tile_om_unit;
  } else {
    const int64_t l16 = lds_for(16);
    const int32_t osu16 = (ob + 15) / 16;
    int32_t g = osu16 * 4, m = 64;
    while (m) { const int32_t r = g % m; g = m; m = r; }  // gcd(osu16 * 4, 64)
    if (l16 <= 64 * 1024 && kLdsPerCu / l16 >= kLdsPerCu / lds4 && g <= 4) omu = 16;
  }
  const int32_t osu = (ob + omu - 1) / omu;
  const int64_t lds = lds_for(omu);
  if (osu > kBlock || lds > 64 * 1024) return false;
  t.ok = 1;
  t.dp = dp; t.gb = gb; t.th = th; t.tw = tw; t.margin = M; t.wh = wh; t.ww = ww;
  t.ps = ps; t.cb = cb; t.osu = osu; t.omu = omu; t.lds_bytes = (int32_t)lds;
  // Rows of a 3x3 kernel (27 values: 56 bytes from the 4-byte boundary below
  // a 16-bit row, 108 bytes of fp32), one group per workgroup: each forward
  // lane reads its own row from global memory into registers, so nothing
  // waits on the staging barrier and the LDS holds the window alone (more
  // workgroups per CU).  Measured on graph-replayed steps: U-Net block
  // 120.7 -> 118.3 us, FlowDCN 115.0 -> 102.8 us, InternImage bf16 45.7 ->
  // 41.5 us, fp32 61.4 -> 57.2 us, wide low-resolution block 62.6 -> 55.2 us.
  const bool can_direct = gb == 1 && d.kernel_h == 3 && d.kernel_w == 3;
  t.om_direct = can_direct && p.tile_om_unit <= 1 ? 1 : 0;
  t.fwd_lds_bytes = t.om_direct
                        ? (int32_t)(((win + 15) & ~int64_t(15)) + (d.dtype == DCN4_BF16 ? 16 : 0))
                        : t.lds_bytes;
  t.slices = slices;
  t.whole = whole ? 1 : 0;
  t.passes = mp;
  t.passes_x = 1;
  if (whole) {
    // tile rows per workgroup: as many as keep at least four workgroups per
    // CU, so that one staging of the image serves more outputs; tile columns
    // only on request (the wide low-resolution block, 2 x 2 tiles per
    // workgroup, 1280 workgroups: 56.5 us against 55.6 us for 2 x 1, 2560
    // workgroups, whose second and third rounds fill the GPU better)
    const int64_t rows = (p.Ho + th - 1) / th, cols = (p.Wo + tw - 1) / tw;
    const int64_t chunks = (int64_t)(d.group / gb) * slices;
    auto wgs = [&](int64_t py, int64_t px) {
      return (int64_t)d.N * ((rows + py - 1) / py) * ((cols + px - 1) / px) * chunks;
    };
    int64_t py = rows, px = p.tile_passes_x > 0 ? p.tile_passes_x : 1;
    if (px > cols) px = cols;
    while (py > 1 && wgs(py, px) < 4 * 256) py = (py + 1) / 2;
    if (p.tile_passes > 0) py = p.tile_passes < rows ? p.tile_passes : rows;
    t.passes = (int32_t)py;
    t.passes_x = (int32_t)px;
  }
  return true;
}

// tile_shape_mp for the plan's margin-window passes (the option, else the
// default; fewer when the window does not fit, never more than the tile rows
// of the output).
bool tile_shape(const Plan& p, int32_t dp, int32_t gb, int32_t slices, bool whole,
                TileShape& t) {
  if (whole) return tile_shape_mp(p, dp, gb, slices, true, 1, t);
  const int32_t lanes_px = gb * (slices > 1 ? 1 : p.D / (dp > 0 ? dp : 1));
  const int32_t tp = lanes_px > 0 && lanes_px <= kBlock ? kBlock / lanes_px : 1;
  int32_t th, tw;
  tile_dims(tp, th, tw);
  const int32_t rows = (p.Ho + th - 1) / th;
  int32_t mp = p.tile_passes > 0 ? p.tile_passes : kDefaultMarginPasses;
  if (mp > rows) mp = rows;
  for (; mp > 1; --mp)
    if (tile_shape_mp(p, dp, gb, slices, false, mp, t)) return true;
  return tile_shape_mp(p, dp, gb, slices, false, 1, t);
}

// The tile shape for one kind of window (see resolve_tile).
TileShape search_tile(const Plan& p, bool whole) {
  const dcn4_desc& d = p.desc;
  // channels per lane: the caller's choice, else the plan's default and then
  // half of it (a smaller tile per lane count keeps wide groups in LDS)
  int32_t dps[2] = {p.dp, 0};
  const int32_t vec = 16 / p.es;
  if (!p.dp_user && p.dp / 2 >= vec && (p.dp / 2) % vec == 0 && p.D % (p.dp / 2) == 0)
    dps[1] = p.dp / 2;
  TileShape t{};
  bool found = false;
  for (int32_t dp : dps) {
    if (dp <= 0) continue;
    if (p.tile_groups > 0) {
      if ((found = tile_shape(p, dp, p.tile_groups, 1, whole, t))) break;
      continue;
    }
    // fewest groups per workgroup that fit: the largest output tile
    for (int32_t gb = 1; gb <= d.group && !found; ++gb)
      if (d.group % gb == 0) found = tile_shape(p, dp, gb, 1, whole, t);
    if (found) break;
  }
  // a group too wide for whole-group windows (its lanes do not divide the
  // workgroup, or its window does not fit): one channel slice per workgroup
  if (!found && p.tile_groups <= 1)
    for (int32_t dp : dps)
      if (dp > 0 && p.D / dp > 1 && (found = tile_shape(p, dp, 1, p.D / dp, whole, t))) break;
  if (!found) t = TileShape{};
  return t;
}

// LDS window bytes a tile shape stages per image: window bytes times
// workgroups per image
double staged_bytes(const Plan& p, const TileShape& t) {
  const int32_t rows = t.th * (t.passes > 0 ? t.passes : 1);  // output rows per workgroup
  const int32_t cols = t.tw * (t.passes_x > 0 ? t.passes_x : 1);  // and columns
  const double tiles = (double)((p.Ho + rows - 1) / rows) * ((p.Wo + cols - 1) / cols);
  const double chunks = (double)(p.desc.group / t.gb) * t.slices;
  return (double)t.wh * t.ww * t.ps * tiles * chunks;
}

}  // namespace

void resolve_tile(Plan& p) {
  const dcn4_desc& d = p.desc;
  p.tile = TileShape{};
  if (p.dp <= 0 || p.kernel_choice == kKernelDirect) return;
  // offset/weight rows must start on 4-byte boundaries (4-byte staging units)
  if ((d.group * 3 * p.K * p.es) % 4) return;
  // The window: the tile's footprint plus the margin (points whose corners
  // leave it take the global path), or the whole image plus a zero border
  // (no point ever leaves it).  Automatic: the whole image when its window
  // fits and stages at most 1.25 times the bytes of the margin window.
  const TileShape tm = p.tile_window == 2 ? TileShape{} : search_tile(p, false);
  const TileShape tw = p.tile_window == 1 ? TileShape{} : search_tile(p, true);
  if (p.tile_window == 1) p.tile = tm;
  else if (p.tile_window == 2) p.tile = tw;
  else if (tw.ok && (!tm.ok || staged_bytes(p, tw) <= 1.25 * staged_bytes(p, tm))) p.tile = tw;
  else p.tile = tm;
}

int32_t tile_f16_window(const Plan& p) {
  const TileShape& ts = p.tile;
  if (!ts.ok || p.desc.dtype != DCN4_BF16 || !p.f16_window) return 0;
  if (p.f16_window == 2) return 2;
  const int32_t cpr = ts.ww * (ts.ps / 16);
  const int32_t wrpp = kBlock / cpr;
  // automatic: through registers when the window fits them; a larger window
  // stays bf16 (re-encoding it in LDS measured slower: FlowDCN tokens 97.0 ->
  // 109.5 us at margin 5, the U-Net block 119.8 -> 121.4 us against the
  // register path)
  return (ts.wh + wrpp - 1) / wrpp <= kF16WinPasses ? 1 : 0;
}

void fill_tile_args(const Plan& p, TileArgs& a) {
  const dcn4_desc& d = p.desc;
  const TileShape& ts = p.tile;
  a.H = d.H; a.W = d.W; a.C = d.C; a.G = d.group; a.D = p.D; a.Ho = p.Ho; a.Wo = p.Wo;
  a.kh = d.kernel_h; a.kw = d.kernel_w; a.sh = d.stride_h; a.sw = d.stride_w;
  a.ph = d.pad_h; a.pw = d.pad_w; a.dh = d.dilation_h; a.dw = d.dilation_w;
  a.offset_scale = d.offset_scale;
  a.Hm1 = (float)(d.H - 1);
  a.Wm1 = (float)(d.W - 1);
  a.L = ts.slices > 1 ? 1 : p.D / ts.dp;
  a.slices = ts.slices;
  a.DSL = ts.slices > 1 ? ts.dp : p.D;
  a.max_scale = d.use_group_scales ? d.max_scale : 0.0f;
  a.swz_shift = p.tile_swizzle > 0 ? p.tile_swizzle - 1 : -1;
  a.GB = ts.gb; a.TH = ts.th; a.TW = ts.tw; a.M = ts.margin;
  a.whole = ts.whole;
  a.passes = ts.passes > 0 ? ts.passes : 1;
  a.passes_x = ts.passes_x > 0 ? ts.passes_x : 1;
  a.WH = ts.wh; a.WW = ts.ww; a.PS = ts.ps; a.CB = ts.cb;
  a.WSQ = ts.whole ? ts.wh : ts.wh - ts.th * (a.passes - 1) * d.stride_h;
  a.cpr = ts.ww * (ts.ps / 16);
  a.wrpp = kBlock / a.cpr;
  a.wpasses = (ts.wh + a.wrpp - 1) / a.wrpp;
  a.OSU = ts.osu;
  a.OMU = ts.omu;
  a.upr = ts.tw * ts.osu;
  if (a.upr <= kBlock) {  // whole tile rows per pass
    a.orpp = kBlock / a.upr;
    a.opasses = (ts.th + a.orpp - 1) / a.orpp;
  } else {                // whole pixels per pass
    a.orpp = 0;
    a.oppp = kBlock / ts.osu;
    a.opasses = (ts.th * ts.tw + a.oppp - 1) / a.oppp;
  }
  a.om_lds = (int32_t)((((int64_t)ts.wh * ts.ww * ts.ps) + 15) & ~int64_t(15));
  a.om_direct = 0;  // set by the forward launch
  a.flag_lds = a.om_lds + ts.th * ts.tw * ts.osu * ts.omu;
  a.f16_window = tile_f16_window(p);
  a.tiles_x = (p.Wo + ts.tw * a.passes_x - 1) / (ts.tw * a.passes_x);
  a.tiles_y = (p.Ho + ts.th * a.passes - 1) / (ts.th * a.passes);
  a.chunks = d.group / ts.gb * ts.slices;
  a.img_bytes = (uint32_t)((uint64_t)d.H * d.W * d.C * p.es);
  a.om_row_bytes = (uint32_t)(d.group * 3 * p.K * p.es);
  a.om_img_bytes = (uint32_t)((uint64_t)p.Ho * p.Wo * a.om_row_bytes);
  a.div_chunks = make_fastdiv((uint32_t)a.chunks);
  a.div_tx = make_fastdiv((uint32_t)a.tiles_x);
  a.div_ty = make_fastdiv((uint32_t)a.tiles_y);
  a.div_cpr = make_fastdiv((uint32_t)a.cpr);
  a.div_cvec = make_fastdiv((uint32_t)(ts.ps / 16));
  a.div_upr = make_fastdiv((uint32_t)a.upr);
  a.div_osu = make_fastdiv((uint32_t)ts.osu);
  a.div_gbl = make_fastdiv((uint32_t)(ts.gb * a.L));
  a.div_L = make_fastdiv((uint32_t)a.L);
  a.div_tw = make_fastdiv((uint32_t)ts.tw);
  a.div_slices = make_fastdiv((uint32_t)ts.slices);
}

dcn4_status launch_tiled(const Plan& p, const void* x, const void* om,
                         const float* scales, const float* pscales, void* y, void* stream) {
  const dcn4_desc& d = p.desc;
  const TileShape& ts = p.tile;
  const int K3 = (d.kernel_h == 3 && d.kernel_w == 3) ? 1 : 0;
  const int nv = ts.dp / (16 / p.es);
  // the pixel stride is a compile-time constant when a lane owns all of an
  // unpadded window pixel (a whole group or a slice; and the window is
  // square: see tile_point)
  const int32_t wsq = ts.whole ? ts.wh : ts.wh - ts.th * (ts.passes - 1) * d.stride_h;
  const bool psc = ts.gb == 1 && (ts.slices > 1 || ts.dp == p.D) && ts.ps == 16 * nv &&
                   wsq == ts.ww;
  const bool whole = ts.whole != 0;
  tile_fn fn = tile_pick(d.dtype, p.mode, nv, K3, psc, whole);
  if (!fn) return DCN4_ERR_UNSUPPORTED;
  TileArgs a{};
  fill_tile_args(p, a);
  a.scales = scales;
  if (ts.om_direct) {  // no offset/weight area: the flag word follows the window
    a.om_direct = 1;
    a.flag_lds = a.om_lds;
  }
  const uint64_t x_img = a.img_bytes, om_img = a.om_img_bytes;
  const uint64_t y_img = (uint64_t)p.Ho * p.Wo * d.C * p.es;
  const uint64_t ps_img = (uint64_t)p.Ho * p.Wo * d.group;  // pixel scales per image
  const int64_t per_image = (int64_t)a.tiles_x * a.tiles_y * a.chunks;
  const int32_t imgs = (int32_t)((int64_t(1) << 30) / per_image);
  for (int32_t n0 = 0; n0 < d.N; n0 += imgs) {
    const int32_t nb = (d.N - n0) < imgs ? (d.N - n0) : imgs;
    a.x = static_cast<const char*>(x) + n0 * x_img;
    a.om = static_cast<const char*>(om) + n0 * om_img;
    a.y = static_cast<char*>(y) + n0 * y_img;
    a.pscales = pscales ? pscales + n0 * ps_img : nullptr;
    a.nblocks = (int32_t)(nb * per_image);
    hipLaunchKernelGGL(fn, dim3(a.nblocks), dim3(kBlock), ts.fwd_lds_bytes,
                       static_cast<hipStream_t>(stream), a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      note_hip_error(e);
      return DCN4_ERR_HIP;
    }
  }
  return DCN4_OK;
}

int32_t backward_lg_shift(int32_t D) {
  int32_t sh = 0;
  while (sh < 4 && (D % (2 << sh)) == 0) ++sh;
  return sh;
}

typedef void (*tile_bwd_fn)(TileArgs, BwdTileArgs);

template <int DT, int MODE, bool SL>
tile_bwd_fn tile_bwd_nv(int nv) {
  constexpr int V = 16 / Io<DT>::es;
  switch (nv) {
    case 1: return dcn4_tile_bwd_kernel<DT, V, 1, MODE, SL>;
    case 2: return dcn4_tile_bwd_kernel<DT, V, 2, MODE, SL>;
    case 3: return dcn4_tile_bwd_kernel<DT, V, 3, MODE, SL>;
    default: return dcn4_tile_bwd_kernel<DT, V, 4, MODE, SL>;
  }
}

// sliced: a workgroup does its group's channel slices in turn
template <int DT, int MODE>
tile_bwd_fn tile_bwd_pick(int nv, bool sliced) {
  return sliced ? tile_bwd_nv<DT, MODE, true>(nv) : tile_bwd_nv<DT, MODE, false>(nv);
}

// LDS bytes of the tiled backward (0: it does not apply to the plan): the
// forward tile's window and offset/weight values.
int32_t tiled_backward_lds(const Plan& p) {
  const dcn4_desc& d = p.desc;
  const TileShape& ts = p.tile;
  if (!ts.ok || d.kernel_h != 3 || d.kernel_w != 3) return 0;
  const int32_t L = ts.slices > 1 ? 1 : p.D / ts.dp;
  if (L != 1 && L != 2 && L != 4) return 0;
  // the write-out reuses the window: a row of 27 floats and an 8-byte base
  // per (pixel, group) item
  const int32_t out_bytes = kBlock / L * (27 * 4 + 8);
  return ts.lds_bytes > out_bytes ? ts.lds_bytes : out_bytes;
}

dcn4_status launch_tiled_backward(const Plan& p, const void* x, const void* om,
                                  const float* scales, const float* pscales, const void* gy,
                                  float* gom, hipStream_t st) {
  const dcn4_desc& d = p.desc;
  const TileShape& ts = p.tile;
  const int nv = ts.dp / (16 / p.es);
  const bool sl = ts.slices > 1;
  tile_bwd_fn fn;
  if (p.mode == kGroupScale)
    fn = d.dtype == DCN4_F32 ? tile_bwd_pick<DCN4_F32, kGroupScale>(nv, sl)
       : d.dtype == DCN4_BF16 ? tile_bwd_pick<DCN4_BF16, kGroupScale>(nv, sl)
                              : tile_bwd_pick<DCN4_F16, kGroupScale>(nv, sl);
  else if (p.mode == kStdScaled)
    fn = d.dtype == DCN4_F32 ? tile_bwd_pick<DCN4_F32, kStdScaled>(nv, sl)
       : d.dtype == DCN4_BF16 ? tile_bwd_pick<DCN4_BF16, kStdScaled>(nv, sl)
                              : tile_bwd_pick<DCN4_F16, kStdScaled>(nv, sl);
  else
    fn = d.dtype == DCN4_F32 ? tile_bwd_pick<DCN4_F32, kStdUnitScale>(nv, sl)
       : d.dtype == DCN4_BF16 ? tile_bwd_pick<DCN4_BF16, kStdUnitScale>(nv, sl)
                              : tile_bwd_pick<DCN4_F16, kStdUnitScale>(nv, sl);
  TileArgs a{};
  fill_tile_args(p, a);
  a.scales = scales;
  a.om_direct = ts.om_direct;  // 16-bit rows of one group: read into registers
  BwdTileArgs b{};
  // one tile row per workgroup (the forward's passes are not used here); a
  // margin window covers that row alone
  if (!ts.whole && a.passes > 1) {
    a.WH = a.WSQ;
    a.wpasses = (a.WH + a.wrpp - 1) / a.wrpp;
  }
  a.passes = 1;
  a.passes_x = 1;
  a.tiles_y = (p.Ho + ts.th - 1) / ts.th;
  a.div_ty = make_fastdiv((uint32_t)a.tiles_y);
  a.tiles_x = (p.Wo + ts.tw - 1) / ts.tw;
  a.div_tx = make_fastdiv((uint32_t)a.tiles_x);
  // a workgroup takes every slice of its group in turn: chunks are groups
  b.nslices = ts.slices;
  a.slices = 1;
  a.div_slices = make_fastdiv(1u);
  a.chunks = d.group / ts.gb;
  a.div_chunks = make_fastdiv((uint32_t)a.chunks);
  const uint64_t x_img = a.img_bytes, om_img = a.om_img_bytes;
  const uint64_t y_img = (uint64_t)p.Ho * p.Wo * d.C * p.es;
  const uint64_t gom_img = (uint64_t)p.Ho * p.Wo * d.group * 3 * p.K;
  const uint64_t ps_img = (uint64_t)p.Ho * p.Wo * d.group;  // pixel scales per image
  const int64_t per_image = (int64_t)a.tiles_x * a.tiles_y * a.chunks;
  const int32_t imgs = (int32_t)((int64_t(1) << 30) / per_image);
  for (int32_t n0 = 0; n0 < d.N; n0 += imgs) {
    const int32_t nb = (d.N - n0) < imgs ? (d.N - n0) : imgs;
    a.x = static_cast<const char*>(x) + n0 * x_img;
    a.om = static_cast<const char*>(om) + n0 * om_img;
    a.pscales = pscales ? pscales + n0 * ps_img : nullptr;
    a.nblocks = (int32_t)(nb * per_image);
    b.gy = static_cast<const char*>(gy) + n0 * y_img;
    b.gom = gom + n0 * gom_img;
    hipLaunchKernelGGL(fn, dim3(a.nblocks), dim3(kBlock), tiled_backward_lds(p), st, a, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      note_hip_error(e);
      return DCN4_ERR_HIP;
    }
  }
  return DCN4_OK;
}

// ------------------------------------------------------------ gathered grad_x: host
// Records per bucket: the mean load of a bucket (K*Ho*Wo samples over
// (H+1)*(W+1) cells) plus three standard deviations of a Poisson count plus
// 4, rounded up to a multiple of 4; samples beyond it take the overflow path.
// The capacity sets the workspace, hence the chunks a bounded workspace
// takes (U-Net block, both gradients, default workspace: capacity 32, five
// chunks, 0.958 ms; 24, 0.868 ms; 20, 0.867 ms; 16, where overflows start
// to cost, 1.005 ms).
uint32_t bucket_capacity(const Plan& p) {
  if (p.bucket_cap > 0) return (uint32_t)p.bucket_cap;
  const dcn4_desc& d = p.desc;
  const double mu = (double)p.K * p.Ho * p.Wo / ((double)(d.H + 1) * (d.W + 1));
  uint32_t cap = (uint32_t)__builtin_ceil(mu + 3.0 * __builtin_sqrt(mu) + 4.0);
  cap = (cap + 3u) & ~3u;
  return cap < 8u ? 8u : cap > 1024u ? 1024u : cap;
}

namespace {

constexpr uint64_t kGatherChunkBytes = uint64_t(2) << 30;  // workspace per launch chunk

uint64_t round256(uint64_t b) { return (b + 255) & ~uint64_t(255); }

// Lanes per (bucket column, group): one per vector of the group, at most 16
// so that a wave spans at least 4 columns
int gather_lanes(int D, int V) {
  const int nchunk = D / V;
  return nchunk < 16 ? nchunk : 16;
}

// The gathered grad_x runs over the batch in chunks of imgs images x gc
// groups.  Workspace of one chunk: [0, 256) the overflow counter; from 256
// the bucket counts (4 bytes per key, (H+1)*(W+1) keys per image and
// group); then the overflow list (4 bytes per sample, Ho*Wo*K per image and
// group); then the records (16 bytes x cap per key).
struct GatherShape {
  bool ok;        // indices of one image fit the kernels' 32-bit counters
  int64_t imgs;   // images per chunk
  int32_t gc;     // groups per chunk
  uint32_t cap;
  uint64_t keys_ig, samples_ig;  // per image and group
  uint64_t list_off, recs_off, bytes;
};

uint64_t chunk_bytes(uint64_t keys_ig, uint64_t samples_ig, uint32_t cap, uint64_t pairs) {
  return 256 + round256(4 * pairs * keys_ig) + round256(4 * pairs * samples_ig) +
         16 * pairs * keys_ig * cap;
}

// Chunks of at most as many (image, group) pairs as fit `budget` bytes of
// workspace (at least one pair, even beyond the budget), as few as possible.
GatherShape gather_shape(const Plan& p, uint64_t budget) {
  GatherShape s{};
  const dcn4_desc& d = p.desc;
  s.cap = bucket_capacity(p);
  s.keys_ig = (uint64_t)(d.H + 1) * (d.W + 1);
  s.samples_ig = (uint64_t)p.Ho * p.Wo * p.K;
  const uint64_t lim = (uint64_t(1) << 31) - 1;
  if (d.N < 1 || s.keys_ig * d.group > lim || s.samples_ig * d.group > lim) return s;
  // pairs per chunk: the budget and the kernels' 32-bit key and sample counts
  uint64_t lo = 1, hi = (uint64_t)d.N * d.group;
  const uint64_t lims[2] = {lim / s.keys_ig, lim / s.samples_ig};
  for (uint64_t c : lims) hi = c < hi ? c : hi;
  while (lo < hi) {  // the largest count that fits
    const uint64_t mid = (lo + hi + 1) / 2;
    if (chunk_bytes(s.keys_ig, s.samples_ig, s.cap, mid) <= budget) lo = mid; else hi = mid - 1;
  }
  const uint64_t pairs = lo;
  // the split into images x groups with the fewest chunks (each chunk is a
  // launch sequence), then the chunks evened out (the smallest workspace for
  // that many chunks)
  uint64_t best_chunks = ~uint64_t(0), best = 0;
  const uint64_t N = (uint64_t)d.N, G = (uint64_t)d.group;
  for (uint64_t gc = G; gc >= 1; --gc) {
    uint64_t imgs = pairs / gc;
    if (imgs > N) imgs = N;
    if (imgs == 0) continue;
    const uint64_t ci = (N + imgs - 1) / imgs, cg = (G + gc - 1) / gc;
    const uint64_t i2 = (N + ci - 1) / ci, g2 = (G + cg - 1) / cg;  // evened out
    if (ci * cg < best_chunks || (ci * cg == best_chunks && i2 * g2 < best)) {
      best_chunks = ci * cg;
      best = i2 * g2;
      s.imgs = (int64_t)i2;
      s.gc = (int32_t)g2;
    }
  }
  s.list_off = 256 + round256(4 * best * s.keys_ig);
  s.recs_off = s.list_off + round256(4 * best * s.samples_ig);
  s.bytes = chunk_bytes(s.keys_ig, s.samples_ig, s.cap, best);
  s.ok = true;
  return s;
}

// Default workspace budget: the operator's ideal traffic bytes, at least one
// (image, group) pair's workspace, at most kGatherChunkBytes.
uint64_t default_gather_budget(const Plan& p) {
  uint64_t b = p.ideal_bytes < kGatherChunkBytes ? p.ideal_bytes : kGatherChunkBytes;
  const GatherShape one = gather_shape(p, 0);
  return one.ok && one.bytes > b ? one.bytes : b;
}

typedef void (*gather_fn)(GatherArgs);

// Output tile of a bucket workgroup (at most kBucketNS samples per thread)
// and the window of cells it counts in LDS: the tile's base rows/cols (the
// centres in group-scale mode, where the grid spreads the points by up to
// (k-1)/2 scaled steps) widened by a margin on each side.
struct BucketTile {
  int32_t TH, tw_shift, WH, WW, wy_off, wx_off;
  int32_t lds_bytes;
};

BucketTile bucket_tile(const Plan& p) {
  const dcn4_desc& d = p.desc;
  static const int shapes[][2] = {{8, 4}, {8, 3}, {4, 3}, {4, 2}, {2, 2}, {2, 1}, {1, 1}, {1, 0}};
  const bool gs = p.mode == kGroupScale;
  const int hy = (d.kernel_h - 1) >> 1, hx = (d.kernel_w - 1) >> 1;
  const int M = gs ? 4 + 4 * (hy > hx ? hy : hx) : 4;
  BucketTile t{};
  for (const auto& sh : shapes) {
    t.TH = sh[0];
    t.tw_shift = sh[1];
    const int TW = 1 << sh[1];
    if (t.TH * TW * p.K > kBucketNS * kBlock) continue;
    if (gs) {
      t.WH = (t.TH - 1) * d.stride_h + 2 * M + 1;
      t.WW = (TW - 1) * d.stride_w + 2 * M + 1;
      t.wy_off = -d.pad_h + hy - M;
      t.wx_off = -d.pad_w + hx - M;
    } else {
      t.WH = (t.TH - 1) * d.stride_h + (d.kernel_h - 1) * d.dilation_h + 2 * M + 1;
      t.WW = (TW - 1) * d.stride_w + (d.kernel_w - 1) * d.dilation_w + 2 * M + 1;
      t.wy_off = -d.pad_h - M;
      t.wx_off = -d.pad_w - M;
    }
    t.lds_bytes = t.WH * t.WW * 4;
    if (t.lds_bytes <= kLdsBudget) return t;
  }
  // windows too large for LDS: every sample takes its slot with its own atomic
  t.WH = t.WW = 1;
  t.wy_off = t.wx_off = -(1 << 30);
  t.lds_bytes = 4;
  return t;
}

template <int DT>
gather_fn pick_bucket(int mode) {
  return mode == kStdUnitScale ? dcn4_bucket_kernel<DT, kStdUnitScale>
       : mode == kStdScaled ? dcn4_bucket_kernel<DT, kStdScaled>
                            : dcn4_bucket_kernel<DT, kGroupScale>;
}

template <int DT, int U>
gather_fn pick_gather_u(bool vec, bool vst, bool stage) {
  constexpr int V = 16 / Io<DT>::es;
  if (!vec) return dcn4_gather_kernel<DT, 1, false, false, U>;
  if (stage)
    return vst ? dcn4_gather_kernel<DT, V, true, true, U> : dcn4_gather_kernel<DT, V, false, true, U>;
  return vst ? dcn4_gather_kernel<DT, V, true, false, U> : dcn4_gather_kernel<DT, V, false, false, U>;
}

// Shape of the gather walk (measured on the workloads): short bands and two
// records per round where occupancy matters more than loads in flight -- a
// staged grad_y window (the window then covers fewer rows and takes less
// LDS) or groups spanning 8 or more lanes (few columns per wave); otherwise
// 8-row bands with 8 records per round.
template <int DT>
gather_fn pick_gather(bool vec, bool vst, bool stage, bool short_band) {
  return short_band ? pick_gather_u<DT, 2>(vec, vst, stage) : pick_gather_u<DT, 8>(vec, vst, stage);
}

// LDS budget of the gather's staged grad_y window: four workgroups per CU.
// Larger windows (64-byte groups: fp32 or D = 32) measured slower staged, at
// two workgroups per CU, than reading grad_y from global memory.
constexpr int kGatherLdsBudget = 40 * 1024;

dcn4_status check_launch() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    note_hip_error(e);
    return DCN4_ERR_HIP;
  }
  return DCN4_OK;
}

dcn4_status launch_gather(const Plan& p, const void* om, const float* scales,
                          const float* pscales, const void* gy, float* gx, void* ws,
                          uint64_t ws_bytes, hipStream_t st) {
  const dcn4_desc& d = p.desc;
  const GatherShape sh = gather_shape(p, ws_bytes < kGatherChunkBytes ? ws_bytes : kGatherChunkBytes);
  const bool vec = p.D % (16 / p.es) == 0 && ((uintptr_t)gy & 15) == 0;
  const bool vst = vec && ((uintptr_t)gx & 15) == 0;
  const int V = vec ? 16 / p.es : 1;
  // grad_y window of a gather workgroup: the output pixels whose samples
  // land in its cells when the displacement is within the margin M
  const int Lg = gather_lanes(p.D, V), Lc = 64 / Lg;
  const bool gsm = p.mode == kGroupScale;
  const int hy = (d.kernel_h - 1) >> 1, hx = (d.kernel_w - 1) >> 1;
  const int M = gsm ? 4 + 4 * (hy > hx ? hy : hx) : 4;
  // the staging test takes the short band's window; without staging, short
  // bands pay only where a wave spans few columns
  const int short_rows = 4, long_rows = 8;
  const int rows_wg = kGatherWaves * short_rows;
  const int oy_off = gsm ? -1 + d.pad_h - hy - M : -1 + d.pad_h - (d.kernel_h - 1) * d.dilation_h - M;
  const int ox_off = gsm ? -1 + d.pad_w - hx - M : -1 + d.pad_w - (d.kernel_w - 1) * d.dilation_w - M;
  const int span_y = rows_wg + 2 * M + (gsm ? 0 : (d.kernel_h - 1) * d.dilation_h);
  const int span_x = Lc - 1 + 2 * M + (gsm ? 0 : (d.kernel_w - 1) * d.dilation_w);
  const int OWH = span_y / d.stride_h + 2, OWW = span_x / d.stride_w + 2;
  const int64_t stage_bytes = (int64_t)OWH * OWW * p.D * p.es;
  const bool stage = vec && stage_bytes <= kGatherLdsBudget;
  const bool short_band = stage || Lg > 4;
  gather_fn bucket, gather;
  typedef void (*overflow_fn)(GatherArgs, int32_t);
  overflow_fn ovf;
  switch (d.dtype) {
    case DCN4_F32:
      bucket = pick_bucket<DCN4_F32>(p.mode);
      gather = pick_gather<DCN4_F32>(vec, vst, stage, short_band);
      ovf = dcn4_overflow_kernel<DCN4_F32>;
      break;
    case DCN4_BF16:
      bucket = pick_bucket<DCN4_BF16>(p.mode);
      gather = pick_gather<DCN4_BF16>(vec, vst, stage, short_band);
      ovf = dcn4_overflow_kernel<DCN4_BF16>;
      break;
    default:
      bucket = pick_bucket<DCN4_F16>(p.mode);
      gather = pick_gather<DCN4_F16>(vec, vst, stage, short_band);
      ovf = dcn4_overflow_kernel<DCN4_F16>;
      break;
  }
  GatherArgs ga{};
  fill_common(p, ga.f);
  ga.f.scales = scales;
  ga.cap = sh.cap;
  ga.K = p.K;
  ga.nchunk = p.D / V;
  ga.Lg = Lg;
  ga.div_K = make_fastdiv((uint32_t)p.K);
  ga.div_kw = make_fastdiv((uint32_t)d.kernel_w);
  ga.gc = sh.gc;
  ga.div_gc = make_fastdiv((uint32_t)sh.gc);
  ga.div_W = make_fastdiv((uint32_t)d.W);
  ga.div_H = make_fastdiv((uint32_t)d.H);
  const BucketTile bt = bucket_tile(p);
  ga.TH = bt.TH;
  ga.tw_shift = bt.tw_shift;
  ga.WH = bt.WH;
  ga.WW = bt.WW;
  ga.wy_off = bt.wy_off;
  ga.wx_off = bt.wx_off;
  ga.tiles_y = (p.Ho + bt.TH - 1) / bt.TH;
  ga.tiles_x = (p.Wo + (1 << bt.tw_shift) - 1) >> bt.tw_shift;
  ga.div_WW = make_fastdiv((uint32_t)bt.WW);
  ga.div_tx = make_fastdiv((uint32_t)ga.tiles_x);
  ga.div_ty = make_fastdiv((uint32_t)ga.tiles_y);
  ga.strips = (d.W + Lc - 2) / (Lc - 1);
  ga.band_rows = short_band ? short_rows : long_rows;
  ga.bands = (d.H + ga.band_rows - 1) / ga.band_rows;
  ga.band_groups = (ga.bands + kGatherWaves - 1) / kGatherWaves;
  ga.div_strips = make_fastdiv((uint32_t)ga.strips);
  ga.div_bgroups = make_fastdiv((uint32_t)ga.band_groups);
  ga.xs = 0;
  while ((1u << ga.xs) < (uint32_t)p.Wo) ++ga.xs;
  ga.OWH = stage ? OWH : 0;
  ga.OWW = stage ? OWW : 1;
  ga.oy_off = oy_off;
  ga.ox_off = ox_off;
  ga.div_OWW = make_fastdiv((uint32_t)ga.OWW);
  ga.div_vpp = make_fastdiv((uint32_t)((p.D * p.es) >> 4 > 0 ? (p.D * p.es) >> 4 : 1));
  const int gather_lds = stage ? (int)stage_bytes : 0;
  char* w = static_cast<char*>(ws);
  ga.listed = reinterpret_cast<uint32_t*>(w);
  ga.counts = reinterpret_cast<uint32_t*>(w + 256);
  ga.list = reinterpret_cast<uint32_t*>(w + sh.list_off);
  ga.recs = reinterpret_cast<u32x4*>(w + sh.recs_off);
  const uint64_t y_img = (uint64_t)p.Ho * p.Wo * d.C * p.es;
  const uint64_t om_img = (uint64_t)p.Ho * p.Wo * d.group * 3 * p.K * p.es;
  const uint64_t ps_img = (uint64_t)p.Ho * p.Wo * d.group;
  const uint64_t x_img = (uint64_t)d.H * d.W * d.C;
  for (int64_t n0 = 0; n0 < d.N; n0 += sh.imgs)
  for (int32_t g0 = 0; g0 < d.group; g0 += sh.gc) {
    const int64_t nb = (d.N - n0) < sh.imgs ? (d.N - n0) : sh.imgs;
    const int32_t gc = (d.group - g0) < sh.gc ? (d.group - g0) : sh.gc;
    ga.g0 = g0;
    ga.gc = gc;
    ga.div_gc = make_fastdiv((uint32_t)gc);
    ga.f.om = static_cast<const char*>(om) + n0 * om_img;
    ga.f.pscales = pscales ? pscales + n0 * ps_img : nullptr;
    ga.gy = static_cast<const char*>(gy) + n0 * y_img;
    ga.gx = gx + n0 * x_img;
    ga.samples = (uint32_t)(nb * gc * sh.samples_ig);
    ga.nblocks = (int32_t)((uint64_t)nb * gc * ga.band_groups * ga.strips);
    const uint64_t zero_words = 64 + (uint64_t)nb * gc * sh.keys_ig;
    const uint64_t zb = (zero_words + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(dcn4_fill_zero_kernel, dim3((unsigned)(zb < 65536 ? zb : 65536)),
                       dim3(kBlock), 0, st, reinterpret_cast<float*>(w), zero_words);
    dcn4_status s = check_launch();
    if (s != DCN4_OK) return s;
    const uint64_t bblocks = (uint64_t)nb * gc * ga.tiles_y * ga.tiles_x;
    hipLaunchKernelGGL(bucket, dim3((unsigned)bblocks), dim3(kBlock), bt.lds_bytes, st, ga);
    if ((s = check_launch()) != DCN4_OK) return s;
    hipLaunchKernelGGL(gather, dim3((unsigned)ga.nblocks), dim3(kBlock), gather_lds, st, ga);
    if ((s = check_launch()) != DCN4_OK) return s;
    const uint64_t ob = ((uint64_t)ga.samples * p.D + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(ovf, dim3((unsigned)(ob < 512 ? ob : 512)), dim3(kBlock), 0, st, ga,
                       (int32_t)p.mode);
    if ((s = check_launch()) != DCN4_OK) return s;
  }
  return DCN4_OK;
}

}  // namespace

uint64_t backward_workspace_bytes(const Plan& p) {
  const GatherShape s = gather_shape(p, default_gather_budget(p));
  return s.ok ? s.bytes : 0;
}

uint64_t backward_min_workspace_bytes(const Plan& p) {
  const GatherShape s = gather_shape(p, 0);
  return s.ok ? s.bytes : 0;
}

// The library's own workspace for callers that cannot allocate
// (dcn4_backward_noalloc): one static device array per GPU, kScratchBytes
// long, held from module load until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); it looks up the array's device address once per device with
// hipGetSymbolAddress, with that device current, and uses that address.
namespace {
__device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

dcn4_status scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    note_hip_error(e);
    return DCN4_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return DCN4_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !q) {
      note_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return DCN4_ERR_HIP;
    }
    g_scratch_ptr[dev] = q;
  }
  *ptr = g_scratch_ptr[dev];
  return DCN4_OK;
}

dcn4_status launch_backward(const Plan& p, const void* x, const void* om,
                            const float* scales, const float* pscales,
                            const void* gy, float* gx, float* gom, void* ws,
                            uint64_t ws_bytes, void* stream, bool vector_path) {
  const dcn4_desc& d = p.desc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (gx && ws) {
    const dcn4_status s = launch_gather(p, om, scales, pscales, gy, gx, ws, ws_bytes, st);
    if (s != DCN4_OK) return s;
    gx = nullptr;  // done: what remains is grad_om
  }
  if (gx) {
    const uint64_t n = (uint64_t)d.N * d.H * d.W * d.C;
    const uint64_t blocks = (n + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(dcn4_fill_zero_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)),
                       dim3(kBlock), 0, st, gx, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      note_hip_error(e);
      return DCN4_ERR_HIP;
    }
  }
  if (!gom && !gx) return DCN4_OK;
  if (!gx && vector_path && p.kernel_choice != kKernelDirect && tiled_backward_lds(p) > 0)
    return launch_tiled_backward(p, x, om, scales, pscales, gy, gom, st);
  const int K3 = (d.kernel_h == 3 && d.kernel_w == 3) ? 1 : 0;
  // grad_offset_mask alone on whole 16-byte vectors: the vector kernel, its
  // rows collected in LDS
  const int nvec = (p.D * p.es) % 16 == 0 ? p.D * p.es / 16 : 0;
  int vec_lg = 0;
  while ((1 << vec_lg) < nvec && vec_lg < 4) ++vec_lg;
  const int om_lds = (kBlock >> vec_lg) * 3 * p.K * 4;
  const bool om_vec = !gx && vector_path && nvec > 0 && om_lds <= kLdsBudget;
  typedef void (*bwd_fn)(BwdArgs);
  bwd_fn fn;
  const int m = p.mode;
#define DCN4_BWD_PICK(KERNEL, DT)                                                      \
  fn = m == kStdUnitScale ? (K3 ? KERNEL<DT, kStdUnitScale, 3>                        \
                                : KERNEL<DT, kStdUnitScale, 0>)                       \
     : m == kStdScaled ? (K3 ? KERNEL<DT, kStdScaled, 3>                               \
                             : KERNEL<DT, kStdScaled, 0>)                              \
                       : (K3 ? KERNEL<DT, kGroupScale, 3>                              \
                             : KERNEL<DT, kGroupScale, 0>)
  switch (d.dtype) {
    case DCN4_F32:
      if (om_vec) DCN4_BWD_PICK(dcn4_backward_om_kernel, DCN4_F32);
      else DCN4_BWD_PICK(dcn4_backward_kernel, DCN4_F32);
      break;
    case DCN4_BF16:
      if (om_vec) DCN4_BWD_PICK(dcn4_backward_om_kernel, DCN4_BF16);
      else DCN4_BWD_PICK(dcn4_backward_kernel, DCN4_BF16);
      break;
    default:
      if (om_vec) DCN4_BWD_PICK(dcn4_backward_om_kernel, DCN4_F16);
      else DCN4_BWD_PICK(dcn4_backward_kernel, DCN4_F16);
      break;
  }
#undef DCN4_BWD_PICK
  BwdArgs b{};
  fill_common(p, b.f);
  b.f.scales = scales;
  b.f.G = d.group;
  b.f.ipp = d.group;
  b.f.div_ipp = make_fastdiv((uint32_t)d.group);
  b.scales = scales;
  b.lg_shift = om_vec ? vec_lg : backward_lg_shift(p.D);
  b.nvec = nvec;
  const int64_t lanes_per_image = (int64_t)p.Ho * p.Wo * d.group << b.lg_shift;
  const uint64_t x_img = (uint64_t)d.H * d.W * d.C * p.es;
  // per launch: lanes below 2^31 and input bytes below 2^31 (32-bit buffer
  // offsets; a single image is validated below 2^31 bytes at plan creation)
  int64_t imgs = ((int64_t(1) << 31) - 1) / lanes_per_image;
  const int64_t imgs_x = (int64_t)(((uint64_t(1) << 31) - 1) / x_img);
  if (imgs_x < imgs) imgs = imgs_x;
  if (imgs < 1) imgs = 1;
  const uint64_t y_img = (uint64_t)p.Ho * p.Wo * d.C * p.es;
  const uint64_t om_img = (uint64_t)p.Ho * p.Wo * d.group * 3 * p.K * p.es;
  const uint64_t ps_img = (uint64_t)p.Ho * p.Wo * d.group;
  for (int64_t n0 = 0; n0 < d.N; n0 += imgs) {
    const int64_t nb = (d.N - n0) < imgs ? (d.N - n0) : imgs;
    b.x = static_cast<const char*>(x) + n0 * x_img;
    b.om = static_cast<const char*>(om) + n0 * om_img;
    b.gy = static_cast<const char*>(gy) + n0 * y_img;
    b.pscales = pscales ? pscales + n0 * ps_img : nullptr;
    b.f.pscales = b.pscales;
    b.gx = gx ? gx + n0 * (uint64_t)d.H * d.W * d.C : nullptr;
    b.gom = gom ? gom + n0 * (uint64_t)p.Ho * p.Wo * d.group * 3 * p.K : nullptr;
    b.x_bytes = nb * x_img;
    b.lanes = nb * lanes_per_image;
    const int64_t blocks = (b.lanes + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kBlock), om_vec ? om_lds : 0, st, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      note_hip_error(e);
      return DCN4_ERR_HIP;
    }
  }
  return DCN4_OK;
}

dcn4_status launch_scale_grads(const Plan& p, const void* x, const void* om,
                               const float* scales, const float* pscales, const void* gy,
                               float* gsg, float* gps, void* stream) {
  const dcn4_desc& d = p.desc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (gsg) {
    hipLaunchKernelGGL(dcn4_fill_zero_kernel, dim3(1), dim3(kBlock), 0, st, gsg,
                       (uint64_t)d.group);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      note_hip_error(e);
      return DCN4_ERR_HIP;
    }
  }
  const int K3 = (d.kernel_h == 3 && d.kernel_w == 3) ? 1 : 0;
  typedef void (*sg_fn)(BwdArgs, float*, float*);
  sg_fn fn;
  switch (d.dtype) {
    case DCN4_F32: fn = K3 ? dcn4_scale_grad_kernel<DCN4_F32, 3> : dcn4_scale_grad_kernel<DCN4_F32, 0>; break;
    case DCN4_BF16: fn = K3 ? dcn4_scale_grad_kernel<DCN4_BF16, 3> : dcn4_scale_grad_kernel<DCN4_BF16, 0>; break;
    default: fn = K3 ? dcn4_scale_grad_kernel<DCN4_F16, 3> : dcn4_scale_grad_kernel<DCN4_F16, 0>; break;
  }
  BwdArgs b{};
  fill_common(p, b.f);
  b.f.scales = scales;
  b.f.G = d.group;
  b.f.ipp = d.group;
  b.f.div_ipp = make_fastdiv((uint32_t)d.group);
  b.scales = scales;
  b.lg_shift = backward_lg_shift(p.D);
  const int64_t lanes_per_image = (int64_t)p.Ho * p.Wo * d.group << b.lg_shift;
  const uint64_t x_img = (uint64_t)d.H * d.W * d.C * p.es;
  int64_t imgs = ((int64_t(1) << 31) - 1) / lanes_per_image;
  const int64_t imgs_x = (int64_t)(((uint64_t(1) << 31) - 1) / x_img);
  if (imgs_x < imgs) imgs = imgs_x;
  if (imgs < 1) imgs = 1;
  const uint64_t y_img = (uint64_t)p.Ho * p.Wo * d.C * p.es;
  const uint64_t om_img = (uint64_t)p.Ho * p.Wo * d.group * 3 * p.K * p.es;
  const uint64_t ps_img = (uint64_t)p.Ho * p.Wo * d.group;
  for (int64_t n0 = 0; n0 < d.N; n0 += imgs) {
    const int64_t nb = (d.N - n0) < imgs ? (d.N - n0) : imgs;
    b.x = static_cast<const char*>(x) + n0 * x_img;
    b.om = static_cast<const char*>(om) + n0 * om_img;
    b.gy = static_cast<const char*>(gy) + n0 * y_img;
    b.pscales = pscales ? pscales + n0 * ps_img : nullptr;
    b.f.pscales = b.pscales;
    b.x_bytes = nb * x_img;
    b.lanes = nb * lanes_per_image;
    const int64_t blocks = (b.lanes + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kBlock), (size_t)d.group * 4, st, b, gsg,
                       gps ? gps + n0 * ps_img : nullptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      note_hip_error(e);
      return DCN4_ERR_HIP;
    }
  }
  return DCN4_OK;
}

dcn4_status launch_probe(const Plan& p, const void* om, const float* scales,
                         const float* pscales, int32_t* y0, int32_t* x0,
                         float* lh, float* lw, uint8_t* inside, void* stream) {
  FwdArgs a{};
  fill_common(p, a);
  a.om = static_cast<const char*>(om);
  a.scales = scales;
  a.pscales = pscales;
  const int64_t count = (int64_t)p.desc.N * p.Ho * p.Wo * p.desc.group * p.K;
  if (count == 0) return DCN4_OK;
  const int64_t blocks = (count + kBlock - 1) / kBlock;
  typedef void (*probe_fn)(FwdArgs, int32_t*, int32_t*, float*, float*, uint8_t*, int64_t);
  probe_fn fn;
  const int m = p.mode;
  switch (p.desc.dtype) {
    case DCN4_F32:
      fn = m == kStdUnitScale ? dcn4_probe_kernel<DCN4_F32, kStdUnitScale>
         : m == kStdScaled ? dcn4_probe_kernel<DCN4_F32, kStdScaled>
                           : dcn4_probe_kernel<DCN4_F32, kGroupScale>;
      break;
    case DCN4_BF16:
      fn = m == kStdUnitScale ? dcn4_probe_kernel<DCN4_BF16, kStdUnitScale>
         : m == kStdScaled ? dcn4_probe_kernel<DCN4_BF16, kStdScaled>
                           : dcn4_probe_kernel<DCN4_BF16, kGroupScale>;
      break;
    default:
      fn = m == kStdUnitScale ? dcn4_probe_kernel<DCN4_F16, kStdUnitScale>
         : m == kStdScaled ? dcn4_probe_kernel<DCN4_F16, kStdScaled>
                           : dcn4_probe_kernel<DCN4_F16, kGroupScale>;
      break;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kBlock), 0,
                     static_cast<hipStream_t>(stream), a, y0, x0, lh, lw,
                     inside, count);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    note_hip_error(e);
    return DCN4_ERR_HIP;
  }
  return DCN4_OK;
}

}  // namespace dcn4
#endif  // DCN4_TILE_PART_DT
