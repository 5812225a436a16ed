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
// Work: a workgroup owns 128 rows x 288 output columns; wave w computes rows
// 32w..32w+31 against 9 column tiles of 32 (144 fp32 accumulators per lane).
// The workgroups of one row block (its column chunks) are consecutive in the
// XCD-aware order, so the second read of the block's features hits the L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn4_internal.h"

namespace dcn4 {

void note_hip_error(hipError_t e);  // dcn4_kernels.hip

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kRows = kLinearRows;  // rows per workgroup (4 waves x 32)
constexpr int kColTiles = 9;        // 32-column tiles per wave
constexpr int kCols = 32 * kColTiles;
static_assert(kRows == 128 && kCols == kLinearCols, "workgroup tile");

__device__ __forceinline__ rsrc_t lin_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ int lin_xcd_block(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + min(x, r) + (b >> 3);
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

template <int DT>
__global__ __launch_bounds__(256) void dcn4_linear_kernel(LinArgs a) {
  const int lb = lin_xcd_block(blockIdx.x, a.nblocks);
  const int bx = lb / a.col_chunks, by = lb - bx * a.col_chunks;
  const int64_t row0 = (int64_t)bx * kRows;
  const int col0 = by * kCols;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int li = l & 31, lk = (l >> 5) * 8;

  // features of this workgroup's rows; rows past M read zeros (range check)
  const int64_t rows_left = a.M - row0;
  const uint64_t fbytes = (uint64_t)rows_left * a.Cin * 2u;
  const rsrc_t fr = lin_rsrc(a.feat + row0 * a.Cin * 2, (uint32_t)(fbytes < 0x7fffffffu ? fbytes : 0x7fffffffu));
  const rsrc_t wr = lin_rsrc(a.weight, a.w_bytes);  // columns past Nout read zeros
  const uint32_t a_off = (uint32_t)((wave * 32 + li) * a.Cin + lk) * 2u;
  uint32_t b_off[kColTiles];
#pragma unroll
  for (int t = 0; t < kColTiles; ++t) b_off[t] = (uint32_t)((col0 + 32 * t + li) * a.Cin + lk) * 2u;

  f32x16 acc[kColTiles];
#pragma unroll
  for (int t = 0; t < kColTiles; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;

  // two register sets used in turn: the fragments of one 16-wide step are in
  // flight while the matrix cores work on the other.  A load past the last
  // step reads the next row's inputs, or zeros past the buffer's range; its
  // products are never issued.
  u32x4 a0f, a1f, b0f[kColTiles], b1f[kColTiles];
  auto load = [&](u32x4& af, u32x4* bf, int k0) {
    const uint32_t kb = (uint32_t)k0 * 2u;
    af = __builtin_amdgcn_raw_buffer_load_b128(fr, (int)(a_off + kb), 0, 0);
#pragma unroll
    for (int t = 0; t < kColTiles; ++t)
      bf[t] = __builtin_amdgcn_raw_buffer_load_b128(wr, (int)(b_off[t] + kb), 0, 0);
  };
  const int steps = a.Cin >> 4;
  load(a0f, b0f, 0);
#pragma unroll 1
  for (int s = 0; s + 1 < steps; s += 2) {
    load(a1f, b1f, 16 * (s + 1));
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) acc[t] = Mfma<DT>::run(a0f, b0f[t], acc[t]);
    load(a0f, b0f, 16 * (s + 2));
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) acc[t] = Mfma<DT>::run(a1f, b1f[t], acc[t]);
  }
  if (steps & 1) {
#pragma unroll
    for (int t = 0; t < kColTiles; ++t) acc[t] = Mfma<DT>::run(a0f, b0f[t], acc[t]);
  }

  // epilogue: bias, round to the I/O dtype, store in om's layout
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
  for (int t = 0; t < kColTiles; ++t) {
    const int col = col0 + 32 * t + li;
    if (col >= a.Nout) continue;
    const float b = a.bias ? a.bias[col] : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t row = row0 + wave * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
      if (row < a.M) out[row * a.Nout + col] = Mfma<DT>::enc(acc[t][e] + b);
    }
  }
}

}  // namespace

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
  a.col_chunks = (Nout + kCols - 1) / kCols;
  const int64_t row_blocks = (M + kRows - 1) / kRows;
  const int64_t blocks = row_blocks * a.col_chunks;
  if (blocks == 0) return DCN4_OK;
  if (blocks > 0x7fffffff) return DCN4_ERR_UNSUPPORTED;
  a.nblocks = (int32_t)blocks;
  void (*fn)(LinArgs) = dtype == DCN4_BF16 ? dcn4_linear_kernel<DCN4_BF16>
                                           : dcn4_linear_kernel<DCN4_F16>;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    note_hip_error(e);
    return DCN4_ERR_HIP;
  }
  return DCN4_OK;
}

}  // namespace dcn4
