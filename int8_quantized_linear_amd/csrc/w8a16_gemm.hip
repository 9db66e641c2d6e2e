// w8a16_gemm.hip — weight-only int8 GEMM for decode on gfx950 (HBM-bound weight streaming).
//
// y[i, j] = w_scale[j] * sum_c x[i, c] * wq[j, c] (+ bias[j]): int8 weights dequantized in
// registers ("Phase 5a: int8 weight-only quantization", Summary; "Day 6 — Quantize It
// Yourself", The mechanism, block 5).  Batch-1 decode is almost all weight streaming
// ("Day 6 — Quantize It Yourself", the question it opens with), so the kernel is built to
// read every weight byte from HBM exactly once at full bandwidth:
//
//   * a workgroup owns 16 output channels and up to 64 activation rows; its 4, 8 or 12
//     wavefronts split the input channels (in-workgroup split-K) so each weight row is
//     streamed by many waves at once, and sum their partial tiles through LDS in a fixed
//     order (deterministic, no atomics);
//   * each wave issues the loads of up to 8 steps of 16 rows x 128 bytes (two 16-byte loads
//     per lane per step) before it converts the first, so 16 KiB per wave are in flight;
//   * when they fit in LDS, the workgroup's activation rows are copied there by
//     direct-to-LDS loads issued before the weight loads, so the weights are the only
//     loads the multiply waits on and each step is multiplied as soon as its own bytes land;
//   * the scale and bias are applied once, after the reduction over k.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant_mma.hpp"
#include "launch.h"
#include "sync.hpp"

namespace i8ql {
namespace {

constexpr int kUnroll = 8;  // steps of k whose loads a wavefront keeps in flight
// The batch a wavefront issues at once: kUnroll steps, or 4 with 12 wavefronts (the longest
// k), where each wavefront walks its 8 steps in two batches.  Measured on MI355X at M = 1:
// 4096 x 12288 12.0 instead of 13.5 us; with 4, 8 or 16 wavefronts, or interleaved steps,
// every decoder shape was as fast or slower.
template <int WAVES>
constexpr int batch_steps() { return WAVES == 12 ? 4 : kUnroll; }
constexpr int kGlobalUnroll = 4;  // the same with activations loaded too (divided by MT)
constexpr size_t kMaxDefaultLds = 65536;  // dynamic LDS usable without a function attribute
constexpr size_t kMaxStageLds = 96 * 1024;  // staged rows up to this much LDS (attribute set)
constexpr size_t kParamTableBytes = 64 * 4;  // the epilogue's scales and biases
constexpr bool kRowKernel = true;  // one activation row: one wavefront per output channel

// Dynamic LDS: the partial tiles of the WAVES wavefronts ([WAVES][MT][64] v4f), then, when
// the activation rows are staged, rows of 2k + 16 bytes (consecutive rows shifted by one
// 16-byte slot, so the row-parallel fragment reads do not collide on banks) and a 16-byte
// zero block.
template <int MT, int WAVES>
constexpr size_t red_bytes() { return static_cast<size_t>(WAVES) * MT * 64 * sizeof(v4f); }

// GS: w_scale holds one scale per (channel, group of 128 input channels), [n, k / 128]; the
// step loop applies them per step (k % 128 == 0) and the epilogue applies bias only.  With
// staged rows the tile's scales are staged too, as an LDS table [step][16 channels] after
// the zero block (one direct-to-LDS dword per lane, issued before everything else).
//
// The epilogue's 16 channel scales and biases are copied to a 64-float LDS table at
// `ptab_off` (the end of the dynamic LDS) by wavefront 0 when the kernel starts, so the
// epilogue reads LDS instead of waiting for a memory round trip after the reduction (loads
// issued as late as their use cost that round trip on every launch).
template <int MT, int WAVES, int YT, bool XLDS, bool GS = false>
__global__ __launch_bounds__(64 * WAVES) void w8a16_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, const float* __restrict__ bias, void* __restrict__ y,
    int64_t m, int64_t n, int64_t k, int ptab_off) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  v4f* red = reinterpret_cast<v4f*>(smem);
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * (16 * MT);
  float* ptab = reinterpret_cast<float*>(smem + ptab_off);
  if (wave == 0) {
    // lanes 0-15: scale of channel n0 + lane (clamped), 16-31: its bias; the other lanes
    // re-read a scale (in bounds, never used).  With group scales the first slot is unused.
    const int64_t c = min(n0 + lane % 16, n - 1);
    const float* src = bias && lane >= 16 && lane < 32 ? bias + c
                                                       : w_scale + c * (GS ? k / kStepK : 1);
    __builtin_amdgcn_global_load_lds(src, ptab, 4, 0, 0);
  }

  const int64_t wr = min(n0 + lane % 16, n - 1);
  const int8_t* wrow = wq + wr * k;
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xok[mt] = m0 + mt * 16 + lane % 16 < m;

  v4f acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
  int sb, se;
  wave_step_range(k, WAVES, wave, sb, se);

  if constexpr (XLDS) {
    // activation copy first, then the first batch of weight loads; wait for the copy only
    // (the weight loads issued after it may stay in flight), then make it visible to all
    char* xs = smem + red_bytes<MT, WAVES>();
    const int rows = static_cast<int>(min(static_cast<int64_t>(16 * MT), m - m0));
    char* xzero = xs + 1024 * stage_insts(rows, k);
    if (threadIdx.x == 0) *reinterpret_cast<v4u*>(xzero) = v4u{0u, 0u, 0u, 0u};
    float* gs = reinterpret_cast<float*>(xzero + 16);
    if constexpr (GS) {
      // instruction i: steps 4i .. 4i + 3 of the 16 channels, lane l -> [4i + l / 16][l % 16]
      const int64_t groups = k / kStepK;
      const int64_t ch = min(n0 + lane % 16, n - 1);
      for (int i = wave; i < static_cast<int>((groups + 3) / 4); i += WAVES) {
        const int64_t st = min(static_cast<int64_t>(4 * i + lane / 16), groups - 1);
        __builtin_amdgcn_global_load_lds(w_scale + ch * groups + st, gs + 64 * i, 4, 0, 0);
      }
    }
    stage_rows<WAVES>(x + m0 * k, nullptr, 1, rows, k, xs);
    asm volatile("" ::: "memory");  // the weight loads stay behind the copy (wait count below)
    __builtin_amdgcn_sched_barrier(0);
    constexpr int U = batch_steps<WAVES>();
    v4u w[U][2];
    load_weight_batch<U>(wrow, k, sb, se, w);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(2 * U, 0));
    bare_barrier();
    const int64_t pitch = 2 * k + 16;
    const char* xrow[MT];
    bool live[MT];
    v4u xb[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = mt * 16 + lane % 16;
      live[mt] = r < rows;
      xrow[mt] = xs + (live[mt] ? r : 0) * pitch;
#pragma unroll
      for (int c = 0; c < 4; ++c) xb[mt][c] = v4u{0u, 0u, 0u, 0u};
    }
    mma_batch_lds<MT, U, GS>(w, xrow, live, xzero, k, sb, se, xb, acc, gs);
    for (int s = sb + U; s < se; s += U) {
      load_weight_batch<U>(wrow, k, s, se, w);
      __builtin_amdgcn_sched_barrier(0);
      mma_batch_lds<MT, U, GS>(w, xrow, live, xzero, k, s, se, xb, acc, gs);
    }
  } else {
    const uint16_t* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      xrow[mt] = x + (xok[mt] ? m0 + mt * 16 + lane % 16 : 0) * k;
    const float* gsr[4];
    if constexpr (GS) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        gsr[r] = w_scale + min(n0 + 4 * (lane / 16) + r, n - 1) * (k / kStepK);
    }
    dequant_mma_steps<MT, (kGlobalUnroll / MT > 0 ? kGlobalUnroll / MT : 1), GS>(
        wrow, xrow, xok, k, sb, se, acc, gsr);
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = acc[mt];
  __syncthreads();
  if (wave != 0) return;

  // Channels 4*(lane/16) + r of the tile, activation row lane % 16 of each m-tile.
  const int64_t nc = n0 + 4 * (lane / 16);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));  // this wave's table copy has landed
  float sc[4], bs[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc[r] = GS ? 1.0f : ptab[4 * (lane / 16) + r];  // group scales were applied per step
    bs[r] = bias ? ptab[16 + 4 * (lane / 16) + r] : 0.0f;
  }
  // the 4 channels of a lane are adjacent: one 8-byte (bf16) or 16-byte (float32) store
  // when they are all real and the output row offsets keep it aligned
  constexpr int kES = YT == I8QL_F32 ? 4 : 2;
  const bool vec_store = n % 4 == 0 && reinterpret_cast<uintptr_t>(y) % (4 * kES) == 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    v4f s = red[mt * 64 + lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) s += red[(w * MT + mt) * 64 + lane];
    const int64_t row = m0 + mt * 16 + lane % 16;
    if (row >= m) continue;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = s[r] * sc[r];
      if (bias) v[r] = v[r] + bs[r];
    }
    if (vec_store && nc + 3 < n) {
      if constexpr (YT == I8QL_F32) {
        *reinterpret_cast<v4f*>(static_cast<float*>(y) + row * n + nc) =
            v4f{v[0], v[1], v[2], v[3]};
      } else {
        const uint32_t lo =
            f32_to_bf16_rne(v[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
        const uint32_t hi =
            f32_to_bf16_rne(v[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + row * n + nc) = make_uint2(lo, hi);
      }
      continue;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t c = nc + r;
      if (c >= n) continue;
      if constexpr (YT == I8QL_F32) {
        static_cast<float*>(y)[row * n + c] = v[r];
      } else {
        static_cast<uint16_t*>(y)[row * n + c] = f32_to_bf16_rne(v[r]);
      }
    }
  }
}

// ---- one activation row (batch-1 decode) ------------------------------------------------
// With a 16-row tile a wavefront can multiply nothing until all 16 rows' bytes of a step have
// landed, and a row's bytes arrive from its own memory channel at its own time, so the
// multiplies of a launch pile up after the last bytes.  With one activation row the matrix
// cores would also use one of their 16 columns.  Here a wavefront owns one output channel:
// each load instruction reads 1 KiB of the row (8 whole 128-byte lines), every load of the
// row is in flight at once (up to kRowChunks 16-byte chunks per lane, k <= 64 * 16 *
// kRowChunks), the codes expand exactly to bf16 (as in dequant_mma.hpp) and meet the bf16
// activations in v_dot2_f32_bf16 (two exact products and their sum into the float32
// accumulator), then the lanes' sums are added by a butterfly of shuffles (fixed order,
// deterministic) and the channel's scale and bias are applied once.  A wavefront finishes as
// soon as its own row is in.  Longer rows (k > 8192) keep the tiled kernel: there its
// batches of loads kept more of each row in flight and ran faster than one wavefront holding
// 12 or 16 chunks per lane.
constexpr int kRowChunks = 8;
typedef short v2s __attribute__((ext_vector_type(2)));  // a bf16 pair, as the builtin takes it

template <int KC, int YT, bool GS>
__global__ __launch_bounds__(256) void w8a16_row_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, const float* __restrict__ bias, void* __restrict__ y,
    int64_t n, int64_t k) {
  const int lane = threadIdx.x % 64;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (row >= n) return;  // (uniform over the wavefront)
  const int64_t chunks = k / 16;
  const v4u* wr = reinterpret_cast<const v4u*>(wq + row * k);
  const v4u* xr = reinterpret_cast<const v4u*>(x);  // 8 activations per 16 bytes
  // each wavefront reads the activations itself (every wavefront reads the same 2k bytes, so
  // they come from the caches); a chunk's codes and its 16 activations are loaded together
  v4u w[KC], xv[KC][2];
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int64_t c = lane + 64 * static_cast<int64_t>(i);
    const int64_t cc = c < chunks ? c : 0;  // in bounds; multiplied by nothing below
    w[i] = wr[cc];
    xv[i][0] = xr[2 * cc];
    xv[i][1] = xr[2 * cc + 1];
  }
  // GS: the scale of each chunk's group of 128 input channels (8 chunks; the 8 lanes
  // 8j .. 8j + 7 hold one group's chunks at each i)
  float gsc[GS ? KC : 1];
  if constexpr (GS) {
    const float* srow = w_scale + row * (k / 128);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int64_t c = lane + 64 * static_cast<int64_t>(i);
      gsc[i] = srow[(c < chunks ? c : 0) / 8];
    }
  }
  asm volatile("" ::: "memory");  // the loads stay here, in order, ahead of every use
  __builtin_amdgcn_sched_barrier(0);
  // every chunk is multiplied (a chunk past the row's end by zero activations), so the loads
  // keep their issue order and each chunk waits only for its own
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const uint32_t in = lane + 64 * i < chunks ? 0xffffffffu : 0u;
    v8bf a[2];
    i8x16_to_bf16(w[i], a[0], a[1]);
    float part = GS ? 0.0f : acc;  // GS: this chunk's products alone
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4u xm = xv[i][h] & in;
      const v4u av = __builtin_bit_cast(v4u, a[h]);
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w};  // bf16 pairs of codes
      const uint32_t xw[4] = {xm.x, xm.y, xm.z, xm.w};  // bf16 pairs of activations
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2s, aw[e]),
                                               __builtin_bit_cast(v2s, xw[e]), part, false);
    }
    if constexpr (GS) {
      // the group's sum over its 8 lanes, times the group's scale, added by the group's
      // first lane
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      part += __shfl_xor(part, 4, 64);
      acc += lane % 8 == 0 ? part * gsc[i] : 0.0f;
    } else {
      acc = part;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane != 0) return;
  float v = GS ? acc : acc * w_scale[row];
  if (bias) v = v + bias[row];
  if constexpr (YT == I8QL_F32) {
    static_cast<float*>(y)[row] = v;
  } else {
    static_cast<uint16_t*>(y)[row] = f32_to_bf16_rne(v);
  }
}

template <int YT, bool GS>
bool launch_row(const void* x, const int8_t* wq, const float* w_scale, const float* bias,
                void* y, int64_t n, int64_t k, hipStream_t stream, hipError_t* err) {
  const int64_t per_lane = (k / 16 + 63) / 64;
  const dim3 grid(static_cast<unsigned>((n + 3) / 4));
  const auto* xx = static_cast<const uint16_t*>(x);
#define I8QL_ROW(KC)                                                                         \
  hipLaunchKernelGGL((w8a16_row_kernel<KC, YT, GS>), grid, dim3(256), 0, stream, xx, wq,      \
                     w_scale, bias, y, n, k)
  if (per_lane <= 4) {
    I8QL_ROW(4);
  } else if (per_lane <= kRowChunks) {
    I8QL_ROW(8);
  } else {
    return false;
  }
#undef I8QL_ROW
  *err = hipGetLastError();
  return true;
}

template <int MT, int WAVES, int YT, bool GS>
hipError_t launch_waves(const void* x, const int8_t* wq, const float* w_scale,
                        const float* bias, void* y, int64_t m, int64_t n, int64_t k,
                        hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + 15) / 16),
                  static_cast<unsigned>((m + 16 * MT - 1) / (16 * MT)));
  const auto* xx = static_cast<const uint16_t*>(x);
  const int rows = static_cast<int>(min(static_cast<int64_t>(16 * MT), m));
  const size_t rbytes = red_bytes<MT, WAVES>();
  const size_t gs_bytes = GS ? 256 * static_cast<size_t>((k / kStepK + 3) / 4) : 0;
  const size_t xlds_tab = rbytes + 1024 * static_cast<size_t>(stage_insts(rows, k)) + 16 + gs_bytes;
  const size_t xlds = xlds_tab + kParamTableBytes;
  // (with more than 16 KiB of partial tiles, the rows of the k that calls for that many
  // waves never fit)
  constexpr bool can_stage = red_bytes<MT, WAVES>() <= kMaxDefaultLds / 4;
  if (can_stage && xlds <= kMaxStageLds) {
    constexpr auto kern = w8a16_kernel<MT, WAVES, YT, can_stage, GS>;
    if (xlds > kMaxDefaultLds) {  // e.g. 8 rows of k = 4096: 70 KiB
      const hipError_t e = allow_dynamic_lds<kern>(static_cast<int>(kMaxStageLds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, grid, dim3(64 * WAVES), xlds, stream, xx, wq, w_scale, bias, y, m,
                       n, k, static_cast<int>(xlds_tab));
  } else {
    hipLaunchKernelGGL((w8a16_kernel<MT, WAVES, YT, false, GS>), grid, dim3(64 * WAVES),
                       rbytes + kParamTableBytes, stream, xx, wq, w_scale, bias, y, m, n, k,
                       static_cast<int>(rbytes));
  }
  return hipGetLastError();
}

// Wavefronts per workgroup: the fewest of 4, 8 and 12 with which each streams at most
// kUnroll steps of k (with 4 or 8, all its loads in flight at once; a wave with fewer real
// steps than kUnroll still issues kUnroll steps of loads, so the count is matched to the
// steps).  Longer k keeps 12 wavefronts, each walking several batches of batch_steps: 16
// wavefronts of 1024 threads would cap the kernel at 128 registers and spill.  One
// 16-channel tile per workgroup: with N / 16 such workgroups the whole weight matrix is in
// flight in about one occupancy round on 256 CUs for the decoder shapes.
template <int MT, int YT, bool GS>
hipError_t launch_mt(const void* x, const int8_t* wq, const float* w_scale, const float* bias,
                     void* y, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  const int64_t steps = (k + kStepK - 1) / kStepK;
  if (steps <= 4 * kUnroll)
    return launch_waves<MT, 4, YT, GS>(x, wq, w_scale, bias, y, m, n, k, stream);
  if (steps <= 8 * kUnroll)
    return launch_waves<MT, 8, YT, GS>(x, wq, w_scale, bias, y, m, n, k, stream);
  return launch_waves<MT, 12, YT, GS>(x, wq, w_scale, bias, y, m, n, k, stream);
}

template <int YT, bool GS>
hipError_t launch_yt(const void* x, const int8_t* wq, const float* w_scale, const float* bias,
                     void* y, int64_t m, int64_t n, int64_t k, hipStream_t stream) {
  if (m <= 16) return launch_mt<1, YT, GS>(x, wq, w_scale, bias, y, m, n, k, stream);
  if (m <= 32) return launch_mt<2, YT, GS>(x, wq, w_scale, bias, y, m, n, k, stream);
  return launch_mt<4, YT, GS>(x, wq, w_scale, bias, y, m, n, k, stream);
}

// One activation row takes the one-row kernel when its k fits; otherwise the tiled kernel.
template <bool GS>
hipError_t launch_gs(const void* x, const int8_t* wq, const float* w_scale, const float* bias,
                     void* y, i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                     hipStream_t stream) {
  if (m == 1 && kRowKernel) {
    hipError_t err = hipSuccess;
    const bool done =
        y_dtype == I8QL_F32
            ? launch_row<I8QL_F32, GS>(x, wq, w_scale, bias, y, n, k, stream, &err)
            : launch_row<I8QL_BF16, GS>(x, wq, w_scale, bias, y, n, k, stream, &err);
    if (done) return err;
  }
  if (y_dtype == I8QL_F32)
    return launch_yt<I8QL_F32, GS>(x, wq, w_scale, bias, y, m, n, k, stream);
  return launch_yt<I8QL_BF16, GS>(x, wq, w_scale, bias, y, m, n, k, stream);
}

}  // namespace

hipError_t launch_w8a16_gemm(const void* x, const int8_t* wq, const float* w_scale,
                             const float* bias, void* y, i8ql_dtype y_dtype, int64_t m,
                             int64_t n, int64_t k, hipStream_t stream) {
  return launch_gs<false>(x, wq, w_scale, bias, y, y_dtype, m, n, k, stream);
}

hipError_t launch_w8a16_gemm_g128(const void* x, const int8_t* wq, const float* w_scale,
                                  const float* bias, void* y, i8ql_dtype y_dtype, int64_t m,
                                  int64_t n, int64_t k, hipStream_t stream) {
  return launch_gs<true>(x, wq, w_scale, bias, y, y_dtype, m, n, k, stream);
}

}  // namespace i8ql
