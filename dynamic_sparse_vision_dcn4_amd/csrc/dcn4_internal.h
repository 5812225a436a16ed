// dcn4_internal.h -- plan and kernel-argument types shared by the C ABI
// (dcn4_api.cpp) and the gfx950 kernels (dcn4_kernels.hip).
#pragma once

#include <stdint.h>

#include "dcn4.h"

namespace dcn4 {

// Division by a run-time invariant divisor d with one multiply-high, an add
// and a shift ("round-up" method of Granlund & Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994): with s = ceil(log2 d)
// and m = floor(2^32 * (2^s - d) / d) + 1, n / d == (mulhi(n, m) + n) >> s
// for every 0 <= n < 2^31.  The host fills it; the kernels apply it.
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1;
  return FastDiv{d, uint32_t(m), s};
}

enum Mode : int32_t {
  kStdUnitScale = 0,  // standard geometry, offset_scale == 1
  kStdScaled = 1,     // standard geometry, offset_scale != 1
  kGroupScale = 2     // FlowDCN groupwise multi-scale geometry
};

// Threads per workgroup of the forward kernel: 4 wave64s, fewer when the
// offset/weight rows one workgroup stages would exceed the LDS budget.
constexpr int kBlock = 256;
// Tile rows of the forward's margin window that one workgroup takes under one
// staging of their joint window (the option tile_passes overrides it).
constexpr int32_t kDefaultMarginPasses = 1;
constexpr int64_t kLdsPerCu = 160 * 1024;  // LDS of one compute unit (gfx950)
constexpr int kLdsBudget = 48 * 1024;

// Everything a forward launch needs, by value (kernel argument).
struct FwdArgs {
  const char* x;         // input of this launch's first image
  const char* om;        // offset/weight tensor of this launch's first image
  const float* scales;   // [G] fp32 (group-scale mode)
  const float* pscales;  // [pixels, G] fp32 of this launch, or null
  float max_scale;       // > 0: clamp of the effective group scale
  char* y;               // output of this launch's first image
  int32_t H, W, C, G, D, Ho, Wo;
  int32_t kh, kw, sh, sw, ph, pw, dh, dw;
  float offset_scale;
  float Hm1, Wm1;        // H - 1, W - 1
  int32_t L;             // lanes per group (D / D')
  int32_t ipp;           // items (lanes) per output pixel, G * L
  int32_t total_items;   // lanes of this launch, < 2^31
  int32_t nblocks;       // workgroups of this launch
  int32_t block;         // threads (= lane items) per workgroup
  int32_t rowel;         // offset/weight elements per output pixel, G * 3K
  uint32_t img_bytes;    // bytes of one input image, H * W * C * es
  uint64_t x_bytes;      // input bytes of this launch
  uint64_t om_bytes;     // offset/weight bytes of this launch
  FastDiv div_ipp, div_L, div_hw, div_wo;
};

// Arguments of the tiled kernel.  A workgroup owns (image, TH x TW output
// tile, chunk of GB groups); it stages a zero-padded input window of WH x WW
// pixels (the tile's sampling footprint plus a margin of M pixels) and the
// tile's offset/weight values in LDS.
struct TileArgs {
  const char* x;         // input of this launch's first image
  const char* om;        // offset/weight tensor of this launch's first image
  const float* scales;
  const float* pscales;  // [pixels, G] from this launch's first image, or null
  float max_scale;       // group-scale mode: largest scale (0: none)
  char* y;
  int32_t H, W, C, G, D, Ho, Wo;
  int32_t kh, kw, sh, sw, ph, pw, dh, dw;
  float offset_scale, Hm1, Wm1;
  int32_t L;             // lanes per (pixel, group), D / D'
  int32_t swz_shift;     // lane-index bit that swaps a lane's vector pairs (-1: none)
  int32_t GB, TH, TW, M; // groups per workgroup, tile, margin
  int32_t WH, WW;        // window rows, cols
  int32_t WSQ;           // rows of the window one tile row alone stages (WH for the
                         // whole image); the square test of a pass uses this square
  int32_t PS;            // LDS bytes per window pixel (CB, maybe padded)
  int32_t CB;            // window bytes per pixel: GB*D*es, or DSL*es when sliced
  int32_t slices;        // channel slices per group (1: whole groups)
  int32_t whole;         // 1: the window is the whole image plus a 1-pixel zero border
  int32_t passes;        // tile rows per workgroup under one window staging
  int32_t passes_x;      // and tile columns (whole-image window; 1 otherwise)
  int32_t DSL;           // channels per slice (D when not sliced)
  int32_t cpr;           // 16-byte chunks per window row, WW*PS/16 (<= 256)
  int32_t wrpp, wpasses; // window rows per staging pass, passes
  int32_t OSU;           // offset/weight units per tile pixel
  int32_t OMU;           // bytes per offset/weight unit: 4 or 16
  int32_t om_direct;     // 1: forward lanes read their offset/weight rows from
                         // global memory into registers (nothing staged in LDS)
  int32_t upr;           // offset/weight units per tile row, TW*OSU
  int32_t orpp;          // tile rows per offset/weight staging pass (0: by pixels)
  int32_t oppp;          // tile pixels per pass when orpp == 0
  int32_t opasses;       // offset/weight staging passes
  int32_t om_lds;        // byte offset of the offset/weight area in LDS
  int32_t f16_window;    // bf16: the window as fp16 when it converts exactly, re-encoded
                         // through registers (1: wpasses fits them) or in LDS (2); 0 never
  int32_t flag_lds;      // byte offset of 16 bytes of LDS for the workgroup's
                         // agreement on the window encoding
  int32_t tiles_x, tiles_y, chunks, nblocks;
  uint32_t img_bytes;    // H*W*C*es
  uint32_t om_img_bytes; // Ho*Wo*G*3K*es
  uint32_t om_row_bytes; // G*3K*es (a multiple of 4)
  FastDiv div_chunks, div_tx, div_ty, div_cpr, div_cvec, div_upr, div_osu,
      div_gbl, div_L, div_tw, div_slices;
};

typedef void (*tile_fn)(TileArgs);
// The tiled forward kernel of one dtype (0 f32, 1 bf16, 2 f16) and sampling
// mode (Mode) for nv 16-byte vectors per lane, a 3x3 kernel (K3), a
// compile-time pixel stride (psc) and the whole-image window (whole); each
// pair is compiled in a translation unit of its own (dcn4_tile_part.hip).
#define DCN4_TILE_PART_FN_(DT, MODE) tile_part_##DT##_##MODE
#define DCN4_TILE_PART_FN(DT, MODE) DCN4_TILE_PART_FN_(DT, MODE)
tile_fn tile_part_0_0(int nv, int K3, bool psc, bool whole);
tile_fn tile_part_0_1(int nv, int K3, bool psc, bool whole);
tile_fn tile_part_0_2(int nv, int K3, bool psc, bool whole);
tile_fn tile_part_1_0(int nv, int K3, bool psc, bool whole);
tile_fn tile_part_1_1(int nv, int K3, bool psc, bool whole);
tile_fn tile_part_1_2(int nv, int K3, bool psc, bool whole);
tile_fn tile_part_2_0(int nv, int K3, bool psc, bool whole);
tile_fn tile_part_2_1(int nv, int K3, bool psc, bool whole);
tile_fn tile_part_2_2(int nv, int K3, bool psc, bool whole);

// Tile shape a plan resolved (ok == 0: the tiled kernel does not apply).
struct TileShape {
  int32_t ok, dp, gb, th, tw, margin, wh, ww, ps, cb, osu, omu, lds_bytes;
  int32_t slices;  // channel slices per group (one lane per pixel when > 1)
  int32_t whole;   // window = the whole image plus a 1-pixel zero border
  int32_t passes;  // forward: tile rows a workgroup takes under one staging
  int32_t passes_x;  // forward, whole-image window: and tile columns
  int32_t om_direct;      // forward: offset/weight rows read into registers
  int32_t fwd_lds_bytes;  // forward's LDS (lds_bytes less the offset/weight
                          // area when om_direct; the backward stages it)
};

enum KernelChoice : int32_t { kKernelAuto = 0, kKernelDirect = 1, kKernelTiled = 2 };

struct Plan {
  dcn4_desc desc;
  int32_t Ho, Wo, D, K, es;
  Mode mode;
  int32_t dp;           // channels per lane on the vector path
  int32_t dp_default;
  uint64_t ideal_bytes;
  int32_t images_per_launch;  // bounds the per-launch lane count below 2^31
  // options (dcn4_plan_set_option) and the tile shape they resolve to
  int32_t kernel_choice, tile_margin, tile_groups, tile_pad, tile_swizzle;
  int32_t tile_window;   // 0 automatic, 1 tile footprint plus margin, 2 whole image
  int32_t tile_passes;   // whole-image window: tile rows per workgroup (0: automatic)
  int32_t tile_passes_x; // whole-image window: tile columns per workgroup (0: automatic)
  int32_t dp_user;       // 1: channels per lane set by the caller
  int32_t bucket_cap;    // records per bucket of the gathered grad_x (0: automatic)
  int32_t f16_window;    // bf16 tiled forward: 1 = fp16 window when exact (automatic
                         // method), 2 = always re-encoded in LDS, 0 = never
  int32_t tile_om_unit;  // tiled kernels' offset/weight copy unit: 0 automatic, 4, 16
  TileShape tile;
};

// Resolves p.tile from the plan's options (the tiled kernel's shape).
void resolve_tile(Plan& p);
// Whether the plan's tiled forward stages a bf16 window through registers
// and re-encodes it as fp16 when every value converts exactly.
// bf16 tiled forward's window encoding: 0 bf16 only, 1 re-encoded as fp16
// through registers, 2 re-encoded in LDS after the copies (when exact)
int32_t tile_f16_window(const Plan& p);

// Kernel-side entry points (dcn4_kernels.hip).  Arguments are validated by
// the caller; these only shape and enqueue the launches.
dcn4_status launch_forward(const Plan& p, const void* x, const void* om,
                           const float* scales, const float* pscales, void* y,
                           void* stream, bool vector_path);
// DCNv3-style comparison: the softmax pass over each (pixel, group) row's
// weights (rows of at most kDcnv3SoftmaxLds bytes per workgroup in LDS) and
// the one-thread-per-channel aggregation (standard geometry only).
constexpr int32_t kDcnv3SoftmaxLds = 32768;
dcn4_status launch_dcnv3_softmax(const Plan& p, const void* om, void* out, void* stream);
dcn4_status launch_dcnv3(const Plan& p, const void* x, const void* om, void* y, void* stream);
dcn4_status launch_tiled(const Plan& p, const void* x, const void* om,
                         const float* scales, const float* pscales, void* y, void* stream);
dcn4_status launch_probe(const Plan& p, const void* om, const float* scales,
                         const float* pscales, int32_t* y0, int32_t* x0,
                         float* lh, float* lw, uint8_t* inside, void* stream);
// Backward pass: write grad_x (if given) and grad_om (if given); both fp32.
// With a workspace of ws_bytes >= backward_min_workspace_bytes(p) bytes
// (256-byte aligned) grad_x is gathered from per-cell buckets; without one it
// is cleared and accumulated with atomics.
// vector_path: x, offset_mask and grad_y are 16-byte aligned (the tiled
// backward may run).
dcn4_status launch_backward(const Plan& p, const void* x, const void* om,
                            const float* scales, const float* pscales,
                            const void* gy, float* gx, float* gom, void* ws,
                            uint64_t ws_bytes, void* stream, bool vector_path);
// Gradients of the group-scale mode's scales: gsg [G] (cleared here, then
// accumulated with fp32 atomics) and gps [N,Ho,Wo,G] (written), either null.
dcn4_status launch_scale_grads(const Plan& p, const void* x, const void* om,
                               const float* scales, const float* pscales, const void* gy,
                               float* gsg, float* gps, void* stream);
// Workspace of the gathered grad_x (0: a single image's indices exceed the
// kernels' 32-bit counters, so only the atomic path applies): chunks of
// (image, group) pairs within the operator's ideal traffic bytes (at least
// one pair, at most 2 GiB).  A launch given ws_bytes of workspace uses
// chunks as large as fit it; the smallest workspace that works holds one
// (image, group) pair.
uint64_t backward_workspace_bytes(const Plan& p);
uint64_t backward_min_workspace_bytes(const Plan& p);
// The static device workspace of dcn4_backward_noalloc: its size, and its
// address on the current device (looked up once per device).
constexpr uint64_t kScratchBytes = uint64_t(64) << 20;
dcn4_status scratch_address(void** ptr);
// Records per bucket the plan's gathered grad_x uses.
uint32_t bucket_capacity(const Plan& p);
// LDS bytes of the tiled backward (offset/weight gradients only) for the plan,
// 0 when it does not apply.
int32_t tiled_backward_lds(const Plan& p);
// Arguments of the merged offset/weight linear layer (dcn4_linear.hip).
// Offset/weight linear layer, size limit of its 32-bit buffer offsets: the
// weight rows of every column block (Nout rounded up by kLinearCols) and
// kLinearRows + 1 feature rows must stay below 2^31 bytes; both bound the
// K-streamed kernel's blocks (128 pixels x 128 columns) from above.
constexpr int kLinearRows = 256;
constexpr int kLinearCols = 128;
// Cin up to which each wave keeps its pixels' features in registers
constexpr int kLinearRsMaxCin = 384;
struct LinArgs {
  const char* feat;    // [M, Cin] I/O dtype (16-bit)
  const char* weight;  // [Nout, Cin] I/O dtype
  const float* bias;   // [Nout] fp32, or null
  char* out;           // [M, Nout] I/O dtype
  int64_t M;
  int32_t Cin, Nout;
  uint32_t w_bytes;    // Nout * Cin * 2
  int32_t col_chunks;  // column tiles per pixel block (K-streamed kernel)
  int32_t nblocks;
  int32_t vec_store;   // Nout % 4 == 0 and out 8-byte aligned: 8-byte stores
};
// Depthwise 3x3 convolution (the optional stage before the offset/weight
// layer): a lane per (segment of pixels along a row, VEC channels).
struct DwArgs {
  const char* x;       // [N,H,W,C] I/O dtype
  const char* w;       // [3,3,C] I/O dtype
  const float* bias;   // [C] fp32, or null
  char* out;           // [N,H,W,C] I/O dtype
  int32_t H, W, C, cv; // cv: channel vectors per pixel, C / VEC
  int32_t segs;        // pixel segments per row
  int64_t lanes;
  int32_t nblocks;
};
dcn4_status launch_dwconv(const void* x, const void* w, const float* bias, void* out,
                          int32_t N, int32_t H, int32_t W, int32_t C, int32_t dtype,
                          bool vector_path, void* stream);
dcn4_status launch_linear(const void* feat, const void* weight, const float* bias,
                          void* out, int64_t M, int32_t Cin, int32_t Nout, int32_t dtype,
                          void* stream);
// Text of the last HIP error a launch reported on this thread.
const char* last_hip_error();
// LDS bytes one forward workgroup of `block` lanes stages (the offset/weight
// rows of its pixels), and the block size a plan uses (0: rows too large).
int32_t forward_lds_bytes(const Plan& p, int32_t lanes_per_group, int32_t block);
int32_t forward_block(const Plan& p, int32_t lanes_per_group);

}  // namespace dcn4

struct dcn4_plan {
  dcn4::Plan p;
};
