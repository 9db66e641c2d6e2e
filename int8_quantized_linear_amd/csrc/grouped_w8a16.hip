// grouped_w8a16.hip — one launch of weight-only int8 GEMMs over routed experts (gfx950).
//
// "Phase 5a: int8 weight-only quantization" (Summary) runs a mixture-of-experts block as a
// single grouped GEMM over expert weights that are stacked into one tensor per projection,
// with per-output-channel int8 codes.  Here the expert-grouped dispatch happens inside the
// kernel: workgroup (tile, e) covers 16 output channels of expert e.  Wavefront 0 scans the
// routing ids in order (loads batched, ballot + prefix popcount, so the row list is
// deterministic) and
// collects the assignments p = token * topk + slot routed to e into an LDS list; a
// workgroup whose list is empty exits at once, so only the experts that received tokens
// cost HBM bytes.  The listed rows are then processed in passes of up to 8: each pass
// copies its (gathered) activation rows into LDS with direct-to-LDS loads issued ahead of
// the weight loads, and runs the dense weight-only GEMM's inner loop (split-K across the
// wavefronts, every weight load of a wave in flight at once, live-row-only fragment reads,
// ordered reduction through LDS).  The extra row of workgroups (e == num_experts) collects
// assignments whose id is outside [0, num_experts) and writes zeros for them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant_mma.hpp"
#include "launch.h"
#include "sync.hpp"

namespace i8ql {
namespace {

constexpr int kUnroll = 8;  // steps of k whose weight loads a wavefront keeps in flight
constexpr int kList = 1024;     // assignments held in LDS per scan window
constexpr int kScanBatch = 8;   // 64-id groups whose loads a scan keeps in flight together
constexpr int kMaxPassRows = 8;  // activation rows staged in LDS per pass

template <int WAVES>
constexpr size_t red_bytes() { return static_cast<size_t>(WAVES) * 64 * sizeof(v4f); }

// Dynamic LDS: [WAVES][64] v4f partial tiles, the staged rows of one pass (pass_rows rows,
// see stage_rows), a 16-byte zero block.
__host__ __device__ inline size_t xs_bytes(int pass_rows, int64_t k) {
  return 1024 * static_cast<size_t>(stage_insts(pass_rows, k)) + 16;
}

template <int WAVES, int YT>
__global__ __launch_bounds__(64 * WAVES) void grouped_w8a16_kernel(
    const uint16_t* __restrict__ x, int x_per_assignment, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t num_experts, const int32_t* __restrict__ ids,
    int64_t total, int64_t topk, void* __restrict__ y, int64_t n, int64_t k, int pass_rows) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int list[kList];
  __shared__ int s_count;
  __shared__ int64_t s_next;
  v4f* red = reinterpret_cast<v4f*>(smem);
  char* xs = smem + red_bytes<WAVES>();
  char* xzero = xs + 1024 * stage_insts(pass_rows, k);

  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  // Expert blocks are dispatched from the highest id down: always-on shared experts are
  // appended after the routed ones and receive every token, so they start first instead of
  // forming the tail (T = 64, MoE 16B gate: 122 -> 94 us).  The extra invalid-id row comes
  // first and normally exits at once.
  const int64_t e = static_cast<int64_t>(gridDim.y) - 1 - blockIdx.y;
  const bool invalid_row = (e == num_experts);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  if (threadIdx.x == 0) *reinterpret_cast<v4u*>(xzero) = v4u{0u, 0u, 0u, 0u};
  // This lane's 4 output-channel scales (wavefront 0 applies them), requested before the
  // scan so that their latency overlaps it.
  const int64_t nc = n0 + 4 * (lane / 16);
  float sc[4] = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0 && !invalid_row) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = w_scale[e * n + min(nc + r, n - 1)];
  }

  int64_t p_next = 0;
  while (true) {
    // ---- expert-grouped dispatch: collect the next window of assignments for e --------
    // The ids are read kScanBatch * 64 at a time, every load of a batch in flight at once
    // (one memory round trip per batch instead of one per 64 ids), then matched 64 at a time
    // in order.
    if (wave == 0) {
      int base = 0;
      int64_t p = p_next;
      bool full = false;
      while (p < total && !full) {
        int32_t idv[kScanBatch];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
          idv[j] = -1;
          if (p + 64 * j < total) {  // groups past the end are neither loaded nor matched
            const int64_t q = p + 64 * j + lane;
            idv[j] = ids[q < total ? q : total - 1];
          }
        }
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
          const int64_t mine = p + lane;
          if (p >= total) break;
          const int32_t id = idv[j];
          const bool match =
              mine < total && (invalid_row ? (id < 0 || id >= num_experts) : (id == e));
          const uint64_t mask = __ballot(match);
          const int cnt = __popcll(mask);
          if (base + cnt > kList) {  // the window is full; resume at p next time
            full = true;
            break;
          }
          if (match) {
            const uint64_t below = lane == 0 ? 0ull : (mask & ((~0ull) >> (64 - lane)));
            list[base + __popcll(below)] = static_cast<int>(mine);
          }
          base += cnt;
          p += 64;
        }
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
      const int64_t pitch = 2 * k + 16;
      const int div = x_per_assignment ? 1 : static_cast<int>(topk);
      int sb, se;
      wave_step_range(k, WAVES, wave, sb, se);
      for (int g = 0; g < count; g += pass_rows) {
        // Activation rows of this pass first, then the first batch of weight loads (a later
        // pass re-reads the same weights, from cache); wait for the rows only (the weight
        // loads issued after them may stay in flight), then publish them to every
        // wavefront.  The compiler barriers keep the weight loads behind the copy, which the
        // wait count relies on.
        const int rows = min(pass_rows, count - g);
        stage_rows<WAVES>(x, list + g, div, rows, k, xs);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        v4u w[kUnroll][2];
        load_weight_batch<kUnroll>(wrow, k, sb, se, w);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * kUnroll, 0));
        bare_barrier();
        const char* xrow[1];
        bool live[1];
        v4u xb[1][4];
        live[0] = lane % 16 < rows;
        xrow[0] = xs + (live[0] ? lane % 16 : 0) * pitch;
#pragma unroll
        for (int c = 0; c < 4; ++c) xb[0][c] = v4u{0u, 0u, 0u, 0u};
        v4f acc[1] = {v4f{0.f, 0.f, 0.f, 0.f}};
        mma_batch_lds<1, kUnroll>(w, xrow, live, xzero, k, sb, se, xb, acc);
        for (int s = sb + kUnroll; s < se; s += kUnroll) {
          load_weight_batch<kUnroll>(wrow, k, s, se, w);
          __builtin_amdgcn_sched_barrier(0);
          mma_batch_lds<1, kUnroll>(w, xrow, live, xzero, k, s, se, xb, acc);
        }
        red[wave * 64 + lane] = acc[0];
        __syncthreads();
        if (wave == 0 && lane % 16 < rows) {
          v4f sum = red[lane];
#pragma unroll
          for (int w2 = 1; w2 < WAVES; ++w2) sum += red[w2 * 64 + lane];
          const int64_t row = list[g + lane % 16];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t c = nc + r;
            if (c >= n) continue;
            const float v = sum[r] * sc[r];
            if constexpr (YT == I8QL_F32) {
              static_cast<float*>(y)[row * n + c] = v;
            } else {
              static_cast<uint16_t*>(y)[row * n + c] = f32_to_bf16_rne(v);
            }
          }
        }
        __syncthreads();  // the staged rows and red[] are reused by the next pass
      }
    }
    if (p_next >= total) break;
    __syncthreads();  // the next window overwrites list[]
  }
}

template <int WAVES, int YT>
hipError_t launch_waves(const void* x, int x_per_assignment, const int8_t* wq,
                        const float* w_scale, int64_t num_experts, const int32_t* ids,
                        int64_t t, int64_t topk, void* y, int64_t n, int64_t k,
                        hipStream_t stream) {
  auto kern = grouped_w8a16_kernel<WAVES, YT>;
  // Rows staged per pass: an expert that each token picks at most once receives at most t
  // rows; one that receives more takes more passes (any count is handled).
  const int pass_rows = static_cast<int>(min(static_cast<int64_t>(kMaxPassRows), t));
  const size_t lds = red_bytes<WAVES>() + xs_bytes(pass_rows, k);
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>((n + 15) / 16), static_cast<unsigned>(num_experts + 1));
  hipLaunchKernelGGL(kern, grid, dim3(64 * WAVES), lds, stream,
                     static_cast<const uint16_t*>(x), x_per_assignment, wq, w_scale,
                     num_experts, ids, t * topk, topk, y, n, k, pass_rows);
  return hipGetLastError();
}

// Wavefronts per workgroup: the fewest of 1, 2, 4 and 8 with which each streams at most
// kUnroll steps of k (one batch of loads in flight), 8 beyond.
template <int YT>
hipError_t launch_yt(const void* x, int x_per_assignment, const int8_t* wq,
                     const float* w_scale, int64_t num_experts, const int32_t* ids, int64_t t,
                     int64_t topk, void* y, int64_t n, int64_t k, hipStream_t stream) {
  const int64_t steps = (k + kStepK - 1) / kStepK;
  if (steps <= kUnroll)
    return launch_waves<1, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t, topk, y,
                               n, k, stream);
  if (steps <= 2 * kUnroll)
    return launch_waves<2, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t, topk, y,
                               n, k, stream);
  if (steps <= 4 * kUnroll)
    return launch_waves<4, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t, topk, y,
                               n, k, stream);
  return launch_waves<8, YT>(x, x_per_assignment, wq, w_scale, num_experts, ids, t, topk, y, n,
                             k, stream);
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
