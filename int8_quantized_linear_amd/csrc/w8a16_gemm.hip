// w8a16_gemm.hip — weight-only int8 GEMM for decode on gfx950 (HBM-bound weight streaming).
//
// y[i, j] = w_scale[j] * sum_c x[i, c] * wq[j, c] (+ bias[j]): int8 weights dequantized in
// registers ("Phase 5a: int8 weight-only quantization", Summary; "Day 6 — Quantize It
// Yourself", The mechanism, block 5).  Batch-1 decode is almost all weight streaming
// ("Day 6 — Quantize It Yourself", the question it opens with), so the kernel is built to
// read every weight byte from HBM exactly once at full bandwidth:
//
//   * a workgroup owns 16 output channels and up to 64 activation rows; its 4, 8 or 16
//     wavefronts split the input channels (in-workgroup split-K) so each weight row is
//     streamed by many waves at once, and sum their partial tiles through LDS in a fixed
//     order (deterministic, no atomics);
//   * each wave issues the loads of up to 8 steps of 16 rows x 128 bytes (two 16-byte loads
//     per lane per step) before it converts the first, so 16 KiB per wave are in flight;
//   * the scale and bias are applied once, after the reduction over k.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant_mma.hpp"
#include "launch.h"

namespace i8ql {
namespace {

constexpr int kUnroll = 8;  // steps of k whose loads a wavefront keeps in flight

template <int MT, int WAVES, int YT>
__global__ __launch_bounds__(64 * WAVES) void w8a16_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, const float* __restrict__ bias, void* __restrict__ y,
    int64_t m, int64_t n, int64_t k) {
  __shared__ v4f red[WAVES][MT][64];
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);

  const int64_t wr = min(n0 + lane % 16, n - 1);
  const int8_t* wrow = wq + wr * k;
  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t r = m0 + mt * 16 + lane % 16;
    xok[mt] = r < m;
    xrow[mt] = x + (xok[mt] ? r : 0) * k;
  }

  v4f acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  int sb, se;
  wave_step_range(k, WAVES, wave, sb, se);
  dequant_mma_steps<MT, kUnroll>(wrow, xrow, xok, k, sb, se, acc);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[wave][mt][lane] = acc[mt];
  __syncthreads();
  if (wave != 0) return;

  // Channels 4*(lane/16) + r of the tile, activation row lane % 16 of each m-tile.
  const int64_t nc = n0 + 4 * (lane / 16);
  float sc[4], bs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t c = min(nc + r, n - 1);
    sc[r] = w_scale[c];
    bs[r] = bias ? bias[c] : 0.0f;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    v4f s = red[0][mt][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) s += red[w][mt][lane];
    const int64_t row = m0 + mt * 16 + lane % 16;
    if (row >= m) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t c = nc + r;
      if (c >= n) continue;
      float v = s[r] * sc[r];
      if (bias) v = v + bs[r];
      if constexpr (YT == I8QL_F32) {
        static_cast<float*>(y)[row * n + c] = v;
      } else {
        static_cast<uint16_t*>(y)[row * n + c] = f32_to_bf16_rne(v);
      }
    }
  }
}

// Wavefronts per workgroup: enough that each streams at most kUnroll steps of k (all its
// loads in flight at once), between 4 and 16.  One 16-channel tile per workgroup; with
// N / 16 workgroups of this size the whole weight matrix is in flight in about one
// occupancy round on 256 CUs for the decoder shapes.
template <int MT, int YT>
hipError_t launch_mt(const void* x, const int8_t* wq, const float* w_scale, const float* bias,
                     void* y, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + 15) / 16),
                  static_cast<unsigned>((m + 16 * MT - 1) / (16 * MT)));
  const int64_t steps = (k + kStepK - 1) / kStepK;
  const auto* xx = static_cast<const uint16_t*>(x);
  if (steps <= 4 * kUnroll) {
    hipLaunchKernelGGL((w8a16_kernel<MT, 4, YT>), grid, dim3(64 * 4), 0, stream, xx, wq, w_scale,
                       bias, y, m, n, k);
  } else if (steps <= 8 * kUnroll) {
    hipLaunchKernelGGL((w8a16_kernel<MT, 8, YT>), grid, dim3(64 * 8), 0, stream, xx, wq, w_scale,
                       bias, y, m, n, k);
  } else {
    hipLaunchKernelGGL((w8a16_kernel<MT, 16, YT>), grid, dim3(64 * 16), 0, stream, xx, wq,
                       w_scale, bias, y, m, n, k);
  }
  return hipGetLastError();
}

template <int YT>
hipError_t launch_yt(const void* x, const int8_t* wq, const float* w_scale, const float* bias,
                     void* y, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (m <= 16) return launch_mt<1, YT>(x, wq, w_scale, bias, y, m, n, k, stream);
  if (m <= 32) return launch_mt<2, YT>(x, wq, w_scale, bias, y, m, n, k, stream);
  return launch_mt<4, YT>(x, wq, w_scale, bias, y, m, n, k, stream);
}

}  // namespace

hipError_t launch_w8a16_gemm(const void* x, const int8_t* wq, const float* w_scale,
                             const float* bias, void* y, i8ql_dtype y_dtype, int64_t m,
                             int64_t n, int64_t k, hipStream_t stream) {
  if (y_dtype == I8QL_F32)
    return launch_yt<I8QL_F32>(x, wq, w_scale, bias, y, m, n, k, stream);
  return launch_yt<I8QL_BF16>(x, wq, w_scale, bias, y, m, n, k, stream);
}

}  // namespace i8ql
