// grouped_w8a16.hip — one launch of weight-only int8 GEMMs over routed experts (gfx950).
//
// "Phase 5a: int8 weight-only quantization" (Summary) runs a mixture-of-experts block as a
// single grouped GEMM over expert weights that are stacked into one tensor per projection,
// with per-output-channel int8 codes.  Here the expert-grouped dispatch happens inside the
// kernel: workgroup (tile, e) covers 16 output channels of expert e.  Wavefront 0 scans the
// routing ids in order (ballot + prefix popcount, so the row list is deterministic) and
// collects the assignments p = token * topk + slot routed to e into an LDS list; a
// workgroup whose list is empty exits at once, so only the experts that received tokens
// cost HBM bytes.  The list is then processed 64 rows at a time with the same dequant-MFMA
// inner loop as the dense weight-only GEMM (split-K across the wavefronts, ordered
// reduction through LDS).  The extra row of workgroups (e == num_experts) collects
// assignments whose id is outside [0, num_experts) and writes zeros for them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant_mma.hpp"
#include "launch.h"

namespace i8ql {
namespace {

constexpr int kUnroll = 4;  // steps per load batch with one m-tile (one step with four)
constexpr int kMT = 4;          // m-tiles of 16 rows per pass
constexpr int kList = 1024;     // assignments held in LDS per scan window

template <int WAVES, int YT>
__global__ __launch_bounds__(64 * WAVES) void grouped_w8a16_kernel(
    const uint16_t* __restrict__ x, int x_per_assignment, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t num_experts, const int32_t* __restrict__ ids,
    int64_t total, int64_t topk, void* __restrict__ y, int64_t n, int64_t k) {
  __shared__ int list[kList];
  __shared__ int s_count;
  __shared__ int64_t s_next;
  __shared__ v4f red[WAVES][kMT][64];

  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int64_t e = blockIdx.y;
  const bool invalid_row = (e == num_experts);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;

  int64_t p_next = 0;
  while (true) {
    // ---- expert-grouped dispatch: collect the next window of assignments for e --------
    if (wave == 0) {
      int base = 0;
      int64_t p = p_next;
      while (p < total) {
        const int64_t mine = p + lane;
        bool match = false;
        if (mine < total) {
          const int32_t id = ids[mine];
          match = invalid_row ? (id < 0 || id >= num_experts) : (id == e);
        }
        const uint64_t mask = __ballot(match);
        const int cnt = __popcll(mask);
        if (base + cnt > kList) break;  // the window is full; resume at p next time
        if (match) {
          const uint64_t below = lane == 0 ? 0ull : (mask & ((~0ull) >> (64 - lane)));
          list[base + __popcll(below)] = static_cast<int>(mine);
        }
        base += cnt;
        p += 64;
      }
      if (lane == 0) {
        s_count = base;
        s_next = p;
      }
    }
    __syncthreads();
    const int count = s_count;
    p_next = s_next;

    if (invalid_row) {
      for (int i = threadIdx.x; i < count * 16; i += 64 * WAVES) {
        const int64_t row = list[i / 16];
        const int64_t c = n0 + i % 16;
        if (c >= n) continue;
        if constexpr (YT == I8QL_F32) {
          static_cast<float*>(y)[row * n + c] = 0.0f;
        } else {
          static_cast<uint16_t*>(y)[row * n + c] = 0;
        }
      }
    } else if (count > 0) {
      const int64_t wr = min(n0 + lane % 16, n - 1);
      const int8_t* wrow = wq + (e * n + wr) * k;
      const int64_t nc = n0 + 4 * (lane / 16);
      for (int g = 0; g < count; g += 16 * kMT) {
        const uint16_t* xrow[kMT];
        bool xok[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const int li = g + mt * 16 + lane % 16;
          xok[mt] = li < count;
          const int64_t p = xok[mt] ? list[li] : 0;
          xrow[mt] = x + (x_per_assignment ? p : p / topk) * k;
        }
        v4f acc[kMT];
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
        int sb, se;
        wave_step_range(k, WAVES, wave, sb, se);
        const int live = min(kMT, (count - g + 15) / 16);
        if (live == 1) {
          const uint16_t* one[1] = {xrow[0]};
          const bool one_ok[1] = {xok[0]};
          v4f a1[1] = {acc[0]};
          dequant_mma_steps<1, kUnroll>(wrow, one, one_ok, k, sb, se, a1);
          acc[0] = a1[0];
        } else {
          dequant_mma_steps<kMT, 1>(wrow, xrow, xok, k, sb, se, acc);
        }
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) red[wave][mt][lane] = acc[mt];
        __syncthreads();
        if (wave == 0) {
          float sc[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[r] = w_scale[e * n + min(nc + r, n - 1)];
#pragma unroll
          for (int mt = 0; mt < kMT; ++mt) {
            const int li = g + mt * 16 + lane % 16;
            if (li >= count) continue;
            v4f s = red[0][mt][lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) s += red[w][mt][lane];
            const int64_t row = list[li];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int64_t c = nc + r;
              if (c >= n) continue;
              const float v = s[r] * sc[r];
              if constexpr (YT == I8QL_F32) {
                static_cast<float*>(y)[row * n + c] = v;
              } else {
                static_cast<uint16_t*>(y)[row * n + c] = f32_to_bf16_rne(v);
              }
            }
          }
        }
        __syncthreads();  // red[] and list[] are reused
      }
    }
    if (p_next >= total) break;
    __syncthreads();  // the next window overwrites list[]
  }
}

template <int YT>
hipError_t launch_yt(const void* x, int x_per_assignment, const int8_t* wq,
                     const float* w_scale, int64_t num_experts, const int32_t* ids, int64_t t,
                     int64_t topk, void* y, int64_t n, int64_t k, hipStream_t stream) {
  constexpr int WAVES = 8;
  const dim3 grid(static_cast<unsigned>((n + 15) / 16), static_cast<unsigned>(num_experts + 1));
  hipLaunchKernelGGL((grouped_w8a16_kernel<WAVES, YT>), grid, dim3(64 * WAVES), 0, stream,
                     static_cast<const uint16_t*>(x), x_per_assignment, wq, w_scale,
                     num_experts, ids, t * topk, topk, y, n, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_w8a16_gemm(const void* x, int x_per_assignment, const int8_t* wq,
                                     const float* w_scale, int64_t num_experts,
                                     const int32_t* expert_ids, int64_t t, int64_t topk,
                                     void* y, i8ql_dtype y_dtype, int64_t n, int64_t k,
                                     hipStream_t stream) {
  if (y_dtype == I8QL_F32)
    return launch_yt<I8QL_F32>(x, x_per_assignment, wq, w_scale, num_experts, expert_ids, t,
                               topk, y, n, k, stream);
  return launch_yt<I8QL_BF16>(x, x_per_assignment, wq, w_scale, num_experts, expert_ids, t,
                              topk, y, n, k, stream);
}

}  // namespace i8ql
