// w8a8_gemm.hip — int8 x int8 -> int32 GEMM on the gfx950 matrix cores with a fused scale
// epilogue.
//
// W8A8 quantizes both operands to int8 so the product runs on the 8-bit matrix units ("Day
// 6 — Quantize It Yourself", The mechanism, block 5); weights carry one scale per output
// channel and activations one per token, and the output is not quantized
// ("feat(quantization): support compressed-tensors W8A8 and mixed modules", Design and
// Supported Execution Scheme).  Biases follow the output channels (same page, Summary).
//
//   acc[i, j] = sum_c xq[i, c] * wq[j, c]   exact in int32 (k <= 133144)
//   y[i, j]   = ((float)acc * x_scale[i]) * w_scale[j] (+ bias[j]) -> float32 or bf16 (RNE),
//               or acc itself for int32 output.
//
// Both operands are K-contiguous (the nn.Linear [out, in] layout and row-major tokens), so
// a tile of either is a stack of 128-byte row segments.  Block tile BM x BN x 128 bytes;
// each 256-thread workgroup has 4 wavefronts in a 2 x 2 grid and each wavefront a
// (BM/2) x (BN/2) sub-tile of v_mfma_i32_32x32x32_i8 products.  Global -> register loads
// of step t+1 are in flight while step t is multiplied out of LDS (two LDS stages, one
// barrier per step).  LDS rows are padded by 16 bytes so the 16-byte fragment reads of a
// wavefront spread over all banks.  Operand fragments: lane l supplies row l % 32 of the
// 32-row block and 16 consecutive k of the 32-k slice, k offset 16 * (l / 32); A and B use
// the same k assignment, which is all the sum needs.  Accumulator: lane l, register r holds
// row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32 of the 32 x 32 block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace i8ql {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;
constexpr int kPitch = kBK + 16;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <int BM, int BN, int YT>
__global__ __launch_bounds__(256) void w8a8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int8_t* __restrict__ wq, const float* __restrict__ w_scale,
    const float* __restrict__ bias, void* __restrict__ y, int64_t m, int64_t n, int64_t k) {
  constexpr int kThreads = 256;
  constexpr int WTM = BM / 2, WTN = BN / 2;  // wavefront sub-tile
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int kChunksPerRow = kBK / 16;
  constexpr int A_LOADS = BM * kChunksPerRow / kThreads;
  constexpr int B_LOADS = BN * kChunksPerRow / kThreads;
  static_assert(A_LOADS * kThreads == BM * kChunksPerRow, "tile/threads mismatch");
  static_assert(B_LOADS * kThreads == BN * kChunksPerRow, "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) int8_t lds[2][(BM + BN) * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = tid / 64;
  const int wm = wave / 2, wn = wave % 2;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int ktiles = static_cast<int>((k + kBK - 1) / kBK);

  uint4 ra[A_LOADS], rb[B_LOADS];
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);

  auto gload = [&](int kt) {
    const int64_t k0 = static_cast<int64_t>(kt) * kBK;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / kChunksPerRow;
      const int64_t kk = k0 + (c % kChunksPerRow) * 16;
      const int64_t gr = min(m0 + row, m - 1);
      ra[i] = kk < k ? *reinterpret_cast<const uint4*>(xq + gr * k + kk) : zero;
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / kChunksPerRow;
      const int64_t kk = k0 + (c % kChunksPerRow) * 16;
      const int64_t gr = min(n0 + row, n - 1);
      rb[i] = kk < k ? *reinterpret_cast<const uint4*>(wq + gr * k + kk) : zero;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<uint4*>(&lds[buf][(c / kChunksPerRow) * kPitch +
                                          (c % kChunksPerRow) * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<uint4*>(&lds[buf][(BM + c / kChunksPerRow) * kPitch +
                                          (c % kChunksPerRow) * 16]) = rb[i];
    }
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  gload(0);
  sstore(0);
  __syncthreads();

  const int frag_row = lane % 32;
  const int frag_k = 16 * (lane / 32);
  for (int kt = 0; kt < ktiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ktiles) gload(kt + 1);
    const int8_t* la = &lds[buf][0];
    const int8_t* lb = &lds[buf][BM * kPitch];
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
      v4i a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const v4i*>(
            la + (wm * WTM + i * 32 + frag_row) * kPitch + s * 32 + frag_k);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const v4i*>(
            lb + (wn * WTN + j * 32 + frag_row) * kPitch + s * 32 + frag_k);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < ktiles) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- fused epilogue ----------------------------------------------------------------
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t col = n0 + wn * WTN + j * 32 + lane % 32;
    if (col >= n) continue;
    float sw = 0.0f, bj = 0.0f;
    if constexpr (YT != I8QL_I32) {
      sw = w_scale[col];
      if (bias) bj = bias[col];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        if (row >= m) continue;
        const int a = acc[i][j][r];
        if constexpr (YT == I8QL_I32) {
          static_cast<int32_t*>(y)[row * n + col] = a;
        } else {
          float v = __fmul_rn(__fmul_rn(static_cast<float>(a), x_scale[row]), sw);
          if (bias) v = __fadd_rn(v, bj);
          if constexpr (YT == I8QL_F32) {
            static_cast<float*>(y)[row * n + col] = v;
          } else {
            static_cast<uint16_t*>(y)[row * n + col] = f32_to_bf16_rne(v);
          }
        }
      }
    }
  }
}

template <int YT>
hipError_t launch_yt(const int8_t* xq, const float* x_scale, const int8_t* wq,
                     const float* w_scale, const float* bias, void* y, int64_t m, int64_t n,
                     int64_t k, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const dim3 grid(static_cast<unsigned>((n + BN - 1) / BN),
                  static_cast<unsigned>((m + BM - 1) / BM));
  hipLaunchKernelGGL((w8a8_kernel<BM, BN, YT>), grid, dim3(256), 0, stream, xq, x_scale, wq,
                     w_scale, bias, y, m, n, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, const float* bias, void* y,
                            i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                            hipStream_t stream) {
  switch (y_dtype) {
    case I8QL_I32: return launch_yt<I8QL_I32>(xq, x_scale, wq, w_scale, bias, y, m, n, k, stream);
    case I8QL_F32: return launch_yt<I8QL_F32>(xq, x_scale, wq, w_scale, bias, y, m, n, k, stream);
    default: return launch_yt<I8QL_BF16>(xq, x_scale, wq, w_scale, bias, y, m, n, k, stream);
  }
}

}  // namespace i8ql
