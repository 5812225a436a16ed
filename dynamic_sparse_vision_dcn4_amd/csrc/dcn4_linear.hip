// dcn4_linear.hip -- the merged offset/weight linear layer on gfx950 MFMA.
//
// [DCNv4 digest] CSDN "（论文速读）DCNv4：高效可变形卷积算子", "方法3": the
// offsets and the aggregation weights come from one merged linear layer, so
// the op's offset/weight tensor is the product
//   om[r, j] = sum_k feat[r, k] * weight[j, k] + bias[j]
// over the pixels r, with om's row layout [G, 3K] per pixel being the layer's
// output order.  This is the one dense contraction of the method, so it runs
// on the matrix cores: v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation;
// the epilogue adds the bias and rounds to the I/O dtype (nearest even), and
// writes om in the layout the aggregation kernels read.
//
// MFMA 32x32x16 operand layout (checked on the device): lane l holds
// A[l % 32][8*(l / 32) + 0..7] and B[8*(l / 32) + 0..7][l % 32]; element e of
// the result is D[8*(e / 4) + 4*(l / 32) + e % 4][l % 32].  With feat
// row-major [M, Cin] and weight row-major [Nout, Cin] both fragments are one
// 16-byte load of 8 consecutive inputs.
//
// Two kernels.  dcn4_linear_rs_kernel (Cin <= 384): 8 consumer waves each
// keep 32 pixels' features in registers for all of Cin and walk the output
// columns in passes of 64, while 4 producer waves stage each pass's weight
// rows in LDS one pass ahead.  dcn4_linear_gemm_kernel (any other Cin that
// is a multiple of 16): a K-streamed GEMM whose workgroup owns 128 pixels x
// 128 output columns, four consumer waves of 64 x 64 multiplying one 64-wide
// stage of features and weights while four producer waves copy the next
// stage into LDS (two stages).  In both the workgroups of one pixel block
// are consecutive in the XCD-aware order, so the block's features come from
// HBM once and from L2 afterwards.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "dcn4_internal.h"

namespace dcn4 {

void note_hip_error(hipError_t e);  // dcn4_kernels.hip

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;


__device__ __forceinline__ rsrc_t lin_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ int lin_xcd_block(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
}

// 16-bit codecs of the depthwise convolution (bf16/fp16 <-> fp32, round to
// nearest even on the way out).
template <int DT> __device__ __forceinline__ float dw_dec(uint32_t h) {
  if constexpr (DT == DCN4_BF16) return __uint_as_float(h << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
template <int DT> __device__ __forceinline__ uint16_t dw_enc(float f) {
  if constexpr (DT == DCN4_BF16) return __builtin_bit_cast(uint16_t, (__bf16)f);
  else return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int DT> struct Mfma;
template <> struct Mfma<DCN4_BF16> {
  __device__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static uint16_t enc(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
};
template <> struct Mfma<DCN4_F16> {
  __device__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static uint16_t enc(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
};

// buffer-to-LDS loads: lane l's 16 (4) bytes from offset voff of the buffer
// land at dst + 16 l (4 l), dst uniform; offsets past the range write zeros.
// The LDS pointer cast exists only in the device pass.
#define DCN4_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
__device__ __forceinline__ void lds_dma16(rsrc_t r, char* dst, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, DCN4_LDS_PTR(dst), 16, voff, 0, 0, 0);
#endif
}
__device__ __forceinline__ void lds_dma4(rsrc_t r, char* dst, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, DCN4_LDS_PTR(dst), 4, voff, 0, 0, 0);
#endif
}

// s_waitcnt immediates (gfx9 encoding, expcnt and lgkmcnt not waited):
// vmcnt 0, and vmcnt n (n < 16)
constexpr int kWaitVmcnt0 = (7 << 4) | (15 << 8);
constexpr int wait_vmcnt(int n) { return n | (7 << 4) | (15 << 8); }

// K-streamed form for every other Cin (a multiple of 16), in producer and
// consumer waves.  A workgroup owns 128 pixels x 128 output columns; four
// consumer waves own 64 x 64 each (2 x 2 MFMA tiles of 32 x 32).  The k
// dimension streams through two LDS stages of kGmBK inputs: four producer
// waves copy the features and the weights (128 rows each) of the next stage
// straight from L2/HBM into LDS with 16-byte buffer-to-LDS loads while the
// consumers multiply this one, so neither the staging registers nor the
// waits on global loads sit in the waves that issue matrix ops (one barrier
// per stage).  64 KB of LDS: two workgroups per CU, so one workgroup's
// prologue and epilogue overlap the other's stages (measured against 256
// pixels in eight consumer waves with three stages, one workgroup per CU:
// the wide block's 1280 -> 1080 layer 76.2 -> 64.7 us, FlowDCN's 1152 -> 432
// 56.0 -> 57.3 us).  A stage row is the 128 bytes of 64 inputs with its
// 16-byte chunks XOR-swizzled by the row index mod 8 (chunk c of row r at
// position c ^ (r & 7)): the copies write LDS in lane order, so the swizzle is
// applied to the global addresses, and a half-wave's fragment read (32
// consecutive rows, one chunk each) spreads over the bank groups.  Inputs
// past Cin and rows past M or Nout read as zeros.  The weights are the A
// operand, so a lane's results are 4 consecutive output columns of one
// pixel.  The column tiles of one pixel block are consecutive in the
// XCD-aware order, so the block's features are read from HBM once and from
// L2 afterwards.
constexpr int kGmBM = 128, kGmBN = 128, kGmBK = 64;
static_assert(kGmBM <= kLinearRows && kGmBN <= kLinearCols,
              "the API's 32-bit offset limit covers one pixel block and one column block");
constexpr int kGmCons = (kGmBM / 64) * (kGmBN / 64), kGmProd = 4;  // consumer and producer waves
constexpr int kGmThreads = 64 * (kGmCons + kGmProd);
constexpr int kGmStages = 2;
constexpr int kGmAhead = kGmStages - 1;  // stages in flight beyond the one being multiplied
constexpr int kGmRowBytes = kGmBK * 2;                      // one staged row, 128 bytes
constexpr int kGmFBytes = kGmBM * kGmRowBytes;              // features of a stage
constexpr int kGmWBytes = kGmBN * kGmRowBytes;              // weights of a stage
constexpr int kGmStageBytes = kGmFBytes + kGmWBytes;
constexpr int kGmLdsBytes = kGmStages * kGmStageBytes;      // 65,536 B: two workgroups per CU
// copies of 64 x 16 bytes (8 rows) per stage, and per producer wave
constexpr int kGmFCopies = kGmFBytes / 1024, kGmWCopies = kGmWBytes / 1024;
constexpr int kGmCopiesPerProd = (kGmFCopies + kGmWCopies) / kGmProd;
static_assert(kGmFCopies % kGmProd == 0 && kGmWCopies % kGmProd == 0, "copies split evenly");
static_assert(kGmCopiesPerProd < 16, "one stage's copies fit a vmcnt wait immediate");

template <int DT>
__global__ __launch_bounds__(kGmThreads) void dcn4_linear_gemm_kernel(LinArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int lb = lin_xcd_block(blockIdx.x, a.nblocks);
  const int bm = lb / a.col_chunks, bn = lb - bm * a.col_chunks;
  const int64_t row0 = (int64_t)bm * kGmBM;
  const int col0 = bn * kGmBN;
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int Cin = a.Cin;
  const int nk = (Cin + kGmBK - 1) / kGmBK;

  if (wave >= kGmCons) {
    // ---- producer: stages kt = 0, 1 first, then stage kt + 2 while the
    // consumers take stage kt
    // the producer index, made provably wave-uniform: the LDS destination of
    // a buffer-to-LDS copy must be, or the compiler loops over its values
    const int pw = __builtin_amdgcn_readfirstlane(wave - kGmCons);
    const int64_t rows_left = a.M - row0;
    const uint64_t fbytes = (uint64_t)rows_left * Cin * 2u;
    const rsrc_t fr = lin_rsrc(a.feat + row0 * Cin * 2,
                               (uint32_t)(fbytes < 0x7fffffffu ? fbytes : 0x7fffffffu));
    const uint64_t wbytes = (uint64_t)(a.Nout - col0) * Cin * 2u;
    const rsrc_t wr = lin_rsrc(a.weight + (int64_t)col0 * Cin * 2,
                               (uint32_t)(wbytes < 0x7fffffffu ? wbytes : 0x7fffffffu));
    // lane l of copy j writes row 8 j + l / 8, position l % 8, i.e. chunk
    // (l % 8) ^ (row % 8) of that row; the row's offset in the operand
    const int lr = l >> 3, lpos = l & 7;
    const int chunk = lpos ^ lr;  // rows 8 j + lr have row % 8 == lr
    auto issue = [&](int kt) {
      char* st = lds + (kt % kGmStages) * kGmStageBytes;
      const int k = kt * kGmBK + 8 * chunk;
      const bool kin = k < Cin;
#pragma unroll
      for (int i = 0; i < kGmFCopies / kGmProd; ++i) {
        const int j = pw + kGmProd * i;
        const int row = 8 * j + lr;
        lds_dma16(fr, st + j * 1024, kin ? (row * Cin + k) * 2 : (int)0x80000000);
      }
#pragma unroll
      for (int i = 0; i < kGmWCopies / kGmProd; ++i) {
        const int j = pw + kGmProd * i;
        const int row = 8 * j + lr;
        lds_dma16(wr, st + kGmFBytes + j * 1024, kin ? (row * Cin + k) * 2 : (int)0x80000000);
      }
    };
    // The producers' barriers are bare s_barrier: the fence of __syncthreads
    // would make them wait for every copy in flight, the next stage's too.
    // A stage's copies have written LDS once vmcnt says so, and the
    // consumers order their own LDS reads around the same barriers.
    static_assert(kGmAhead == 1 || kGmAhead == 2, "one or two stages ahead");
    issue(0);
    if (kGmAhead == 2 && nk > 1) {
      issue(1);
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(kGmCopiesPerProd));
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    __builtin_amdgcn_s_barrier();  // stage 0 in LDS
    for (int kt = 0; kt < nk; ++kt) {
      // into the buffer of stage kt + kGmAhead - kGmStages = kt - 1, whose
      // reads ended before the last barrier
      if (kt + kGmAhead < nk) {
        issue(kt + kGmAhead);
        if (kGmAhead == 2) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kGmCopiesPerProd));
        else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      }
      __builtin_amdgcn_s_barrier();  // stage kt + 1 has landed
    }
    return;
  }

  // ---- consumer
  const int li = l & 31, h = l >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int tj = 0; tj < 2; ++tj)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tj][tp][e] = 0.0f;
  // fragment rows of this lane: weights wn*64 + 32 t + li, features
  // wm*64 + 32 t + li; their swizzle (row % 8 == li % 8 for both)
  const int sw = li & 7;
  const int wrow = (wn * 64 + li) * kGmRowBytes, frow = (wm * 64 + li) * kGmRowBytes;
  __syncthreads();  // stage 0 in LDS
  for (int kt = 0; kt < nk; ++kt) {
    const char* st = lds + (kt % kGmStages) * kGmStageBytes;
#pragma unroll
    for (int kk = 0; kk < kGmBK; kk += 16) {
      if (kt * kGmBK + kk >= Cin) break;
      const int pos = 16 * (((kk >> 3) + h) ^ sw);
      u32x4 fw[2], ff[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        fw[t] = *reinterpret_cast<const u32x4*>(st + kGmFBytes + wrow + t * 32 * kGmRowBytes + pos);
        ff[t] = *reinterpret_cast<const u32x4*>(st + frow + t * 32 * kGmRowBytes + pos);
      }
#pragma unroll
      for (int tj = 0; tj < 2; ++tj)
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) acc[tj][tp] = Mfma<DT>::run(fw[tj], ff[tp], acc[tj][tp]);
    }
    __syncthreads();  // done with stage kt; stage kt + 1 has landed
  }

  // epilogue: element e of tile (tj, tp) is output column col0 + 64 wn +
  // 32 tj + 8(e/4) + 4h + e%4 of pixel row0 + 64 wm + 32 tp + li
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
  for (int tp = 0; tp < 2; ++tp) {
    const int64_t pix = row0 + wm * 64 + tp * 32 + li;
    if (pix >= a.M) continue;
#pragma unroll
    for (int tj = 0; tj < 2; ++tj) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = col0 + wn * 64 + tj * 32 + 8 * g + 4 * h;
        if (col >= a.Nout) continue;
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float b = (a.bias && col + e < a.Nout) ? a.bias[col + e] : 0.0f;
          v[e] = Mfma<DT>::enc(acc[tj][tp][4 * g + e] + b);
        }
        uint16_t* dst = out + pix * a.Nout + col;
        if (a.vec_store) {
          *reinterpret_cast<u32x2*>(dst) = u32x2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < a.Nout) dst[e] = (uint16_t)v[e];
        }
      }
    }
  }
}

// Register-stationary form for Cin <= 384, in producer/consumer waves.
//
// kRsConsumers consumer waves each own 32 pixels and keep their features for
// every k in registers (Cin/16 fragments).  They walk the output columns in
// passes of two 32-wide tiles (two independent accumulation chains), issue
// the matrix ops and store the results.  kRsProducers producer waves copy each pass's
// weights (2 x 32 rows of Cin, contiguous in the weight matrix) and bias from
// L2 straight into LDS with buffer-to-LDS loads, double-buffered, one pass
// ahead, so the staging holds no registers and every wait on global loads
// sits in the producers (on gfx9 loads and stores share one completion
// counter: a wave that stores outputs and then waits for its own loads also
// waits for its stores).  One wave's buffer-to-LDS loads are bounded by its
// outstanding requests (about 20 GB/s per CU measured); kRsProducers waves
// share each pass.
//
// The weights are the MFMA's A operand: lane (li, h) of a result holds
// pixel li, columns 8(e/4) + 4h + e%4.  LDS weight layout: row j of a tile
// occupies Q + 1 16-byte vectors (Q = Cin/8, one pad vector), so a fragment
// read (32 rows, one vector each) touches distinct bank groups, and the
// producer fills one row per instruction from 640 contiguous bytes.
// Epilogue: each consumer rounds its 32 x 64 outputs into a private LDS area
// (rows of 128 bytes plus 16 bytes of padding) and reads them back so that
// one store instruction writes 4 pixel rows of 128 contiguous bytes.
constexpr int kRsConsumers = 8;                 // consumer waves per workgroup
constexpr int kRsProducers = 4;                 // producer waves per workgroup
constexpr int kRsThreads = 64 * (kRsConsumers + kRsProducers);
constexpr int kRsPixels = 32 * kRsConsumers;    // pixels per workgroup
constexpr int kRsAhead = 2;                     // fragment-read steps kept in flight
constexpr int kRsOutRow = 144;                  // bytes per pixel row of the output area
constexpr int kRsOutBytes = 32 * kRsOutRow;     // one consumer's output area

template <int S> struct RsLayout {
  static constexpr int Q = 2 * S;                 // 16-byte vectors per weight row
  static constexpr int RS = Q + 1;                // padded row stride (vectors)
  static constexpr int kTileBytes = 32 * RS * 16; // one column tile's weights
  static constexpr int kPassBytes = 2 * kTileBytes + 64 * 4;  // + 64 fp32 bias
  static constexpr int kLdsBytes = 2 * kPassBytes + kRsConsumers * kRsOutBytes;
};


template <int DT, int S>
__global__ __launch_bounds__(kRsThreads) void dcn4_linear_rs_kernel(LinArgs a) {
  using L = RsLayout<S>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63, li = l & 31, h = l >> 5;
  const int64_t row0 = (int64_t)blockIdx.x * kRsPixels;
  const int npass = (a.Nout + 63) >> 6;

  if (wave >= kRsConsumers) {
    // producer: a pass's 64 weight rows occupy 64 (Q + 1) consecutive LDS
    // vectors, filled by Q + 1 buffer-to-LDS loads of 64 lanes: lane l of
    // load i fills vector n = 64 i + l, row n / (Q + 1), input vector
    // n % (Q + 1); a pad slot loads the row's last vector again (never read).
    // Rows past Nout read as zeros (range check).
    const rsrc_t wr = lin_rsrc(a.weight, a.w_bytes);
    const rsrc_t br = lin_rsrc(a.bias, a.bias ? (uint32_t)a.Nout * 4u : 0u);
    // the producer index, made provably wave-uniform: the LDS destination of
    // a buffer-to-LDS copy must be, or the compiler loops over its values
    const int pw = __builtin_amdgcn_readfirstlane(wave - kRsConsumers);
    auto issue = [&](int p) {
      char* buf = lds + (p & 1) * L::kPassBytes;
      const int pass_off = p * 64 * L::Q * 16;
#pragma unroll 4
      for (int i = pw; i < L::RS; i += kRsProducers) {
        const int n = 64 * i + l, j = n / L::RS, q = n - j * L::RS;
        lds_dma16(wr, buf + i * 1024, pass_off + (j * L::Q + (q < L::Q ? q : L::Q - 1)) * 16);
      }
      // bias of the pass's 64 columns (zeros past Nout or without bias)
      if (pw == 0) lds_dma4(br, buf + 2 * L::kTileBytes, (p * 64 + l) * 4);
    };
    // the first pass is requested before the consumers request their
    // features, so it does not queue behind them
    issue(0);
    __syncthreads();
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    for (int p = 0; p < npass; ++p) {
      if (p + 1 < npass) issue(p + 1);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    }
    return;
  }

  // consumer: this wave's features, pixels past M read as zeros (requested
  // after the producers have requested the first pass)
  __syncthreads();
  const int64_t rows_left = a.M - row0;
  const uint64_t fbytes = (uint64_t)rows_left * (S * 32u);
  const rsrc_t fr = lin_rsrc(a.feat + row0 * (S * 32),
                             (uint32_t)(fbytes < 0x7fffffffu ? fbytes : 0x7fffffffu));
  u32x4 f[S];
#pragma unroll
  for (int s = 0; s < S; ++s)
    f[s] = __builtin_amdgcn_raw_buffer_load_b128(fr, (wave * 32 + li) * (S * 32) + s * 32 + h * 16,
                                                 0, 0);
  // wait for the features here, once: inside the pass loop the only
  // outstanding global operations are then this wave's stores, which nothing
  // waits for
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  char* ostage = lds + 2 * L::kPassBytes + wave * kRsOutBytes;
  const int64_t pix0 = row0 + wave * 32;
  const bool vec_store = a.vec_store;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  __syncthreads();
  for (int p = 0; p < npass; ++p) {
    const char* cur = lds + (p & 1) * L::kPassBytes;
    const char* wrow = cur + li * (L::RS * 16) + h * 16;
    f32x16 acc0, acc1;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc0[e] = acc1[e] = 0.0f;
    u32x4 w0[S], w1[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      w0[s] = *reinterpret_cast<const u32x4*>(wrow + s * 32);
      w1[s] = *reinterpret_cast<const u32x4*>(wrow + L::kTileBytes + s * 32);
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
      acc0 = Mfma<DT>::run(w0[s], f[s], acc0);
      acc1 = Mfma<DT>::run(w1[s], f[s], acc1);
    }
    // schedule: kRsAhead steps of fragment reads in flight ahead of the
    // matrix ops
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kRsAhead, 0);
#pragma unroll
    for (int s = 0; s < S - kRsAhead; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kRsAhead, 0);

    // epilogue: bias, round, pixel-major rows in this wave's output area
    const float* bl = reinterpret_cast<const float*>(cur + 2 * L::kTileBytes);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x16& acc = t ? acc1 : acc0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cl = 32 * t + 8 * g + 4 * h;
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = Mfma<DT>::enc(acc[4 * g + e] + bl[cl + e]);
        *reinterpret_cast<u32x2*>(ostage + li * kRsOutRow + cl * 2) =
            u32x2{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
      }
    }
    // read back: lane l takes 8 bytes (columns 4(l%16)..+3) of row 4k + l/16
    const int c0 = p * 64 + 4 * (l & 15);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 4 * k + (l >> 4);
      const u32x2 v = *reinterpret_cast<const u32x2*>(ostage + r * kRsOutRow + (l & 15) * 8);
      const int64_t pix = pix0 + r;
      if (pix >= a.M || c0 >= a.Nout) continue;
      uint16_t* dst = out + pix * a.Nout + c0;
      if (vec_store) {
        *reinterpret_cast<u32x2*>(dst) = v;
      } else {
        const uint16_t e4[4] = {(uint16_t)v[0], (uint16_t)(v[0] >> 16), (uint16_t)v[1],
                                (uint16_t)(v[1] >> 16)};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c0 + e < a.Nout) dst[e] = e4[e];
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------ depthwise 3x3 convolution
// The optional stage in front of the offset/weight layer ([DCNv4 digest]
// "方法3": DCNv3's offset subnetwork without its LayerNorm and GELU):
//   out[n,y,x,c] = sum_{i,j<3} w[i,j,c] * x[n, y+i-1, x+j-1, c] + bias[c],
// stride 1, zero padding 1, channel-last.  A lane owns VEC consecutive
// channels (16 bytes on the vector path, one element on the element path) of
// a segment of kDwSeg pixels along a row: it keeps its nine weight vectors in
// registers and slides a 3x3 window of input vectors along the segment, so
// each output needs three new loads, fetched one output ahead.  fp32 fma over the nine taps in
// row-major order, a tap outside the image skipped (so a non-finite weight
// cannot leak into the padding), then the bias, one rounding to the I/O
// dtype.  Consecutive lanes cover a segment's channels, then the next
// segment, so loads and stores of a wave are contiguous runs; the XCD-aware
// block order keeps a band of image rows (the three rows a tap row reads)
// in one XCD's L2.
constexpr int kDwSeg = 16;  // output pixels per lane along a row

// Raw input vector of (row yy, column xs): 16 bytes (vector path) or one
// element widened to its bit pattern (element path); zeros when !in.
template <int DT, int VEC>
__device__ __forceinline__ u32x4 dw_load(const DwArgs& a, int64_t img, int32_t yy, int32_t xs,
                                         int32_t c0, bool in) {
  constexpr int es = DT == DCN4_F32 ? 4 : 2;
  const int64_t off = ((img * a.H + yy) * a.W + xs) * (int64_t)a.C + c0;
  u32x4 r = {0u, 0u, 0u, 0u};
  if (in) {
    if constexpr (VEC > 1) r = *reinterpret_cast<const u32x4*>(a.x + off * es);
    else if constexpr (es == 4) r[0] = reinterpret_cast<const uint32_t*>(a.x)[off];
    else r[0] = reinterpret_cast<const uint16_t*>(a.x)[off];
  }
  return r;
}

// Element e of a raw vector as fp32.
template <int DT, int VEC>
__device__ __forceinline__ float dw_elem(const u32x4& r, int e) {
  if constexpr (DT == DCN4_F32) return __uint_as_float(r[e]);
  else if constexpr (VEC > 1) return dw_dec<DT>((r[e >> 1] >> (16 * (e & 1))) & 0xffffu);
  else return dw_dec<DT>(r[0]);
}

template <int DT, int VEC>
__global__ __launch_bounds__(256) void dcn4_dwconv_kernel(DwArgs a) {
  constexpr int es = DT == DCN4_F32 ? 4 : 2;
  const int lb = lin_xcd_block(blockIdx.x, a.nblocks);
  const int64_t lane = (int64_t)lb * 256 + threadIdx.x;
  if (lane >= a.lanes) return;
  // lane -> (image, row, segment, channel vector)
  const int64_t seg = lane / a.cv;
  const int32_t c0 = (int32_t)(lane - seg * a.cv) * VEC;
  const int64_t row = seg / a.segs;              // n * H + y
  const int32_t x0 = (int32_t)(seg - row * a.segs) * kDwSeg;
  const int64_t img = row / a.H;
  const int32_t y = (int32_t)(row - img * a.H);
  // the nine weight vectors, widened once
  float wv[9][VEC];
#pragma unroll
  for (int t = 0; t < 9; ++t) {
    const int64_t woff = (int64_t)t * a.C + c0;
    u32x4 r = {0u, 0u, 0u, 0u};
    if constexpr (VEC > 1) r = *reinterpret_cast<const u32x4*>(a.w + woff * es);
    else if constexpr (es == 4) r[0] = reinterpret_cast<const uint32_t*>(a.w)[woff];
    else r[0] = reinterpret_cast<const uint16_t*>(a.w)[woff];
#pragma unroll
    for (int e = 0; e < VEC; ++e) wv[t][e] = dw_elem<DT, VEC>(r, e);
  }
  float bv[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) bv[e] = a.bias ? a.bias[c0 + e] : 0.0f;
  const bool row_ok[3] = {y >= 1, true, y + 1 < a.H};
  // raw window columns x-1, x, x+1 of rows y-1, y, y+1; column x+2 is
  // fetched one output ahead
  u32x4 win[3][3], nxt[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    win[i][0] = dw_load<DT, VEC>(a, img, y + i - 1, x0 - 1, c0, row_ok[i] && x0 >= 1);
    win[i][1] = dw_load<DT, VEC>(a, img, y + i - 1, x0, c0, row_ok[i]);
    win[i][2] = dw_load<DT, VEC>(a, img, y + i - 1, x0 + 1, c0, row_ok[i] && x0 + 1 < a.W);
  }
  char* dst = a.out + ((row * a.W + x0) * (int64_t)a.C + c0) * es;
#pragma unroll
  for (int p = 0; p < kDwSeg; ++p) {
    const int32_t x = x0 + p;
    if (x >= a.W) break;
    if (p + 1 < kDwSeg) {
#pragma unroll
      for (int i = 0; i < 3; ++i)
        nxt[i] = dw_load<DT, VEC>(a, img, y + i - 1, x + 2, c0, row_ok[i] && x + 2 < a.W);
    }
    const bool col_ok[3] = {x >= 1, true, x + 1 < a.W};
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (!row_ok[i]) continue;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (!col_ok[j]) continue;
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          acc[e] = __builtin_fmaf(wv[i * 3 + j][e], dw_elem<DT, VEC>(win[i][j], e), acc[e]);
      }
    }
    if (a.bias) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] = acc[e] + bv[e];
    }
    // the empty asm keeps each fp32 sum a value of its own, so the conversion
    // below is a separate rounding (not fused with the last add)
#pragma unroll
    for (int e = 0; e < VEC; ++e) asm volatile("" : "+v"(acc[e]));
    if constexpr (VEC > 1) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (es == 4)
          o[q] = __float_as_uint(acc[q]);
        else
          o[q] = (uint32_t)dw_enc<DT>(acc[2 * q]) | ((uint32_t)dw_enc<DT>(acc[2 * q + 1]) << 16);
      }
      *reinterpret_cast<u32x4*>(dst) = o;
    } else {
      if constexpr (es == 4) *reinterpret_cast<float*>(dst) = acc[0];
      else *reinterpret_cast<uint16_t*>(dst) = dw_enc<DT>(acc[0]);
    }
    dst += (int64_t)a.C * es;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      win[i][0] = win[i][1];
      win[i][1] = win[i][2];
      win[i][2] = nxt[i];
    }
  }
}

// Raises the kernel's dynamic LDS limit to `bytes` on the current device,
// once per kernel and device (the attribute is per-device state).
bool rs_lds_attribute_set(void (*fn)(LinArgs), size_t bytes) {
  constexpr int kMaxDev = 64, kMaxFn = 16;
  static std::atomic<uintptr_t> done[kMaxDev][kMaxFn];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  const uintptr_t key = reinterpret_cast<uintptr_t>(fn);
  std::atomic<uintptr_t>* slot = nullptr;
  if (e == hipSuccess && dev >= 0 && dev < kMaxDev)
    for (int i = 0; i < kMaxFn; ++i) {
      const uintptr_t v = done[dev][i].load(std::memory_order_acquire);
      if (v == key) return true;
      if (v == 0) { slot = &done[dev][i]; break; }
    }
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) {
    note_hip_error(e);
    return false;
  }
  if (slot) {
    uintptr_t expect = 0;
    slot->compare_exchange_strong(expect, key, std::memory_order_acq_rel);
  }
  return true;
}

}  // namespace

dcn4_status launch_dwconv(const void* x, const void* w, const float* bias, void* out,
                          int32_t N, int32_t H, int32_t W, int32_t C, int32_t dtype,
                          bool vector_path, void* stream) {
  DwArgs a{};
  a.x = static_cast<const char*>(x);
  a.w = static_cast<const char*>(w);
  a.bias = bias;
  a.out = static_cast<char*>(out);
  a.H = H; a.W = W; a.C = C;
  const int vec = vector_path ? (dtype == DCN4_F32 ? 4 : 8) : 1;
  a.cv = C / vec;
  a.segs = (W + kDwSeg - 1) / kDwSeg;
  a.lanes = (int64_t)N * H * a.segs * a.cv;
  const int64_t blocks = (a.lanes + 255) / 256;
  if (blocks == 0) return DCN4_OK;
  if (blocks > 0x7fffffff) return DCN4_ERR_UNSUPPORTED;
  a.nblocks = (int32_t)blocks;
  void (*fn)(DwArgs) = nullptr;
  switch (dtype) {
    case DCN4_F32:
      fn = vector_path ? dcn4_dwconv_kernel<DCN4_F32, 4> : dcn4_dwconv_kernel<DCN4_F32, 1>;
      break;
    case DCN4_BF16:
      fn = vector_path ? dcn4_dwconv_kernel<DCN4_BF16, 8> : dcn4_dwconv_kernel<DCN4_BF16, 1>;
      break;
    default:
      fn = vector_path ? dcn4_dwconv_kernel<DCN4_F16, 8> : dcn4_dwconv_kernel<DCN4_F16, 1>;
      break;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    note_hip_error(e);
    return DCN4_ERR_HIP;
  }
  return DCN4_OK;
}

dcn4_status launch_linear(const void* feat, const void* weight, const float* bias,
                          void* out, int64_t M, int32_t Cin, int32_t Nout, int32_t dtype,
                          void* stream) {
  LinArgs a{};
  a.feat = static_cast<const char*>(feat);
  a.weight = static_cast<const char*>(weight);
  a.bias = bias;
  a.out = static_cast<char*>(out);
  a.M = M;
  a.Cin = Cin;
  a.Nout = Nout;
  a.w_bytes = (uint32_t)((int64_t)Nout * Cin * 2);
  a.vec_store = (Nout % 4 == 0) && (reinterpret_cast<uintptr_t>(out) % 8 == 0);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (Cin % 64 == 0 && Cin <= kLinearRsMaxCin) {
    const int64_t blocks = (M + kRsPixels - 1) / kRsPixels;
    if (blocks == 0) return DCN4_OK;
    if (blocks > 0x7fffffff) return DCN4_ERR_UNSUPPORTED;
    void (*fn)(LinArgs) = nullptr;
    size_t lds = 0;
#define DCN4_RS_CASE(n)                                                              \
  case n:                                                                           \
    fn = dtype == DCN4_BF16 ? dcn4_linear_rs_kernel<DCN4_BF16, n>                    \
                            : dcn4_linear_rs_kernel<DCN4_F16, n>;                   \
    lds = RsLayout<n>::kLdsBytes;                                                    \
    break;
    switch (Cin / 16) {
      DCN4_RS_CASE(4) DCN4_RS_CASE(8) DCN4_RS_CASE(12)
      DCN4_RS_CASE(16) DCN4_RS_CASE(20) DCN4_RS_CASE(24)
      default: return DCN4_ERR_UNSUPPORTED;
    }
#undef DCN4_RS_CASE
    if (!rs_lds_attribute_set(fn, lds)) return DCN4_ERR_HIP;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kRsThreads), lds, st, a);
  } else {
    a.col_chunks = (Nout + kGmBN - 1) / kGmBN;
    const int64_t row_blocks = (M + kGmBM - 1) / kGmBM;
    const int64_t blocks = row_blocks * a.col_chunks;
    if (blocks == 0) return DCN4_OK;
    if (blocks > 0x7fffffff) return DCN4_ERR_UNSUPPORTED;
    a.nblocks = (int32_t)blocks;
    void (*fn)(LinArgs) = dtype == DCN4_BF16 ? dcn4_linear_gemm_kernel<DCN4_BF16>
                                             : dcn4_linear_gemm_kernel<DCN4_F16>;
    if (!rs_lds_attribute_set(fn, kGmLdsBytes)) return DCN4_ERR_HIP;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kGmThreads), kGmLdsBytes, st, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    note_hip_error(e);
    return DCN4_ERR_HIP;
  }
  return DCN4_OK;
}

}  // namespace dcn4
