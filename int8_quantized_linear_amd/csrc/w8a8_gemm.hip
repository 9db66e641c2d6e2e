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
// Data movement.  Both operands are K-contiguous (the nn.Linear [out, in] layout and
// row-major tokens).  A workgroup owns a BM x BN output tile and walks k in 64-byte steps.
// Each step's A and B slices are copied global -> LDS by the gfx950 direct-to-LDS loads
// (global_load_lds_dwordx4: 16 bytes per lane, a wavefront fills 1 KiB of LDS = 16 rows x 64
// bytes), so no VGPRs hold staged data and STAGES - 1 future steps stay in flight while the
// current one is multiplied.  Each iteration waits (s_waitcnt vmcnt) for its own step's
// loads, passes one barrier (which also retires the reads of the stage about to be
// refilled), issues the loads of step t + STAGES - 1, then runs the MFMAs.
//
// LDS layout.  A stage holds BM + BN rows of 64 bytes.  The four 16-byte chunks of row r are
// stored XOR-swizzled (physical chunk = logical chunk ^ ((r >> 1) & 3)) so that the 16-byte
// fragment reads of eight consecutive lanes hit eight distinct bank groups; the swizzle is
// applied on the global side (each lane fetches the logical chunk that belongs in its
// fixed LDS slot).
//
// MFMA.  Each wavefront owns a (BM / WAVES_M) x (BN / WAVES_N) sub-tile of 32 x 32 blocks of
// v_mfma_i32_32x32x32_i8.  Fragment layout: lane l supplies row l % 32 of a 32-row block and
// 16 consecutive k of the 32-k slice at offset 16 * (l / 32); A and B use the same k
// assignment, which is all the sum needs.  Accumulator: lane l, register r holds row
// 8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32 of the block.
//
// Tails.  Rows past m or n read a clamped valid row and are never stored.  Chunks past k
// (k % 16 == 0, so chunks are whole) read the row start and are zeroed at fragment-read time
// in the last step.
//
// Configurations: 256 x 256 with 8 wavefronts (128 x 64 each; 4 stages = 128 KiB of LDS,
// one workgroup per CU) when the grid has enough tiles to fill the 256 CUs, else 128 x 128
// with 4 wavefronts (64 x 64 each; 64 KiB, two workgroups per CU).
//
// Tile order.  Consecutive workgroup ids are spread round-robin over the 8 XCDs, each with
// its own L2.  The linear id is remapped so that every XCD receives a contiguous range of
// tiles, walked in groups of GROUP_M tile rows so that neighbouring workgroups share A rows
// and B rows in the XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace i8ql {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;        // bytes of k per step
constexpr int kStages = 4;
constexpr int kRowsPerLoad = 16;  // one wavefront load instruction = 16 rows x 64 bytes
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Linear workgroup id -> (tile row, tile column), XCD-contiguous and grouped.
__device__ __forceinline__ bool tile_of(int64_t tiles_m, int64_t tiles_n, int64_t& tm,
                                        int64_t& tn) {
  const int64_t total = tiles_m * tiles_n;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t b = blockIdx.x;
  const int64_t t = (b % kXcds) * per_xcd + b / kXcds;
  if (t >= total) return false;
  const int64_t group = t / (kGroupM * tiles_n);
  const int64_t first_m = group * kGroupM;
  const int64_t gsize = min(tiles_m - first_m, static_cast<int64_t>(kGroupM));
  const int64_t in_group = t % (kGroupM * tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
  return true;
}

// Wait until at most `pending` of this wavefront's load batches are outstanding, then
// barrier.  The barrier carries no fence: LDS ordering is exactly the vmcnt wait plus the
// MFMAs' own lgkmcnt waits, and the "memory" clobber keeps the compiler from moving LDS
// accesses across it.
template <int LOADS>
__device__ __forceinline__ void wait_and_barrier(int pending) {
  if (pending >= 2) {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * LOADS) : "memory");
  } else if (pending == 1) {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(LOADS) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// Issue this wavefront's direct-to-LDS loads of k step `step` into `stage`.  A chunk past
// the end of the row (k % 16 == 0, so chunks are whole) reads the row start instead, which is
// in bounds; its bytes are zeroed when the fragment is read.
template <int LOADS>
__device__ __forceinline__ void issue_step(int8_t* stage, const int8_t* const* src,
                                           const int* col, const int* dst, int step,
                                           int64_t k) {
  const int64_t k0 = static_cast<int64_t>(step) * kBK;
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int64_t kk = k0 + col[j];
    const int8_t* g = src[j] + (kk < k ? kk : 0);
    __builtin_amdgcn_global_load_lds(g, stage + dst[j], 16, 0, 0);
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int YT>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void w8a8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int8_t* __restrict__ wq, const float* __restrict__ w_scale,
    const float* __restrict__ bias, void* __restrict__ y, int64_t m, int64_t n, int64_t k) {
  constexpr int kWaves = WAVES_M * WAVES_N;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wavefront sub-tile
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int kLoadsA = BM / kRowsPerLoad, kLoadsB = BN / kRowsPerLoad;
  constexpr int LOADS = (kLoadsA + kLoadsB) / kWaves;  // per wavefront per step
  static_assert(LOADS * kWaves == kLoadsA + kLoadsB, "loads must split evenly over waves");
  static_assert(kStages == 4, "wait_and_barrier assumes 4 stages");
  constexpr int kStageBytes = (BM + BN) * kBK;

  extern __shared__ __attribute__((aligned(16))) int8_t lds[];

  int64_t tm, tn;
  if (!tile_of((m + BM - 1) / BM, (n + BN - 1) / BN, tm, tn)) return;
  const int64_t m0 = tm * BM;
  const int64_t n0 = tn * BN;

  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int ksteps = static_cast<int>((k + kBK - 1) / kBK);

  // This lane's part of each of the wavefront's load instructions: instruction j covers tile
  // rows 16 * (wave + kWaves * j) .. +15 of the stacked [A; B] slice.
  const int8_t* src[LOADS];
  int col[LOADS];
  int dst[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int blk = wave + kWaves * j;
    const int trow = blk * kRowsPerLoad + lane / 4;  // row of the stacked tile
    const int pchunk = lane % 4;
    const int lchunk = pchunk ^ ((trow >> 1) & 3);
    col[j] = lchunk * 16;
    if (trow < BM)
      src[j] = xq + min(m0 + trow, m - 1) * k;
    else
      src[j] = wq + min(n0 + (trow - BM), n - 1) * k;
    dst[j] = blk * kRowsPerLoad * kBK;  // wave-uniform LDS offset of the instruction
  }


  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < ksteps) issue_step<LOADS>(lds + s * kStageBytes, src, col, dst, s, k);

  const int frow = lane % 32;
  const int fx = (frow >> 1) & 3;  // swizzle of this lane's fragment rows
  const int a_off = (wm * WTM + frow) * kBK;
  const int b_off = (BM + wn * WTN + frow) * kBK;

  for (int t = 0; t < ksteps; ++t) {
    wait_and_barrier<LOADS>(min(kStages - 1, ksteps - t) - 1);
    if (t + kStages - 1 < ksteps) {
      const int nt = t + kStages - 1;
      issue_step<LOADS>(lds + (nt % kStages) * kStageBytes, src, col, dst, nt, k);
    }
    const int8_t* stage = lds + (t % kStages) * kStageBytes;
    const bool tail = static_cast<int64_t>(t + 1) * kBK > k;
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
      const int lchunk = 2 * s + lane / 32;
      const int pofs = ((lchunk ^ fx) * 16);
      const bool live = !tail || static_cast<int64_t>(t) * kBK + lchunk * 16 < k;
      v4i a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        a[i] = *reinterpret_cast<const v4i*>(stage + a_off + i * 32 * kBK + pofs);
        if (!live) a[i] = v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const v4i*>(stage + b_off + j * 32 * kBK + pofs);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- fused epilogue ----------------------------------------------------------------
  const int64_t row_base = m0 + wm * WTM + 4 * (lane / 32);
  const int64_t col_base = n0 + wn * WTN + lane % 32;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t c = col_base + j * 32;
    if (c >= n) continue;
    float sw = 0.0f, bj = 0.0f;
    if constexpr (YT != I8QL_I32) {
      sw = w_scale[c];
      if (bias) bj = bias[c];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row_base + i * 32 + 8 * (r / 4) + r % 4;
        if (row >= m) continue;
        const int a = acc[i][j][r];
        if constexpr (YT == I8QL_I32) {
          static_cast<int32_t*>(y)[row * n + c] = a;
        } else {
          float v = __fmul_rn(__fmul_rn(static_cast<float>(a), x_scale[row]), sw);
          if (bias) v = __fadd_rn(v, bj);
          if constexpr (YT == I8QL_F32) {
            static_cast<float*>(y)[row * n + c] = v;
          } else {
            static_cast<uint16_t*>(y)[row * n + c] = f32_to_bf16_rne(v);
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int YT>
hipError_t launch_cfg(const int8_t* xq, const float* x_scale, const int8_t* wq,
                      const float* w_scale, const float* bias, void* y, int64_t m, int64_t n,
                      int64_t k, hipStream_t stream) {
  auto kern = w8a8_kernel<BM, BN, WM, WN, YT>;
  constexpr size_t lds = static_cast<size_t>(kStages) * (BM + BN) * kBK;
  static bool configured = false;  // idempotent attribute set; a race only repeats it
  if (!configured) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(lds));
    if (e != hipSuccess) return e;
    configured = true;
  }
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(64 * WM * WN), lds, stream,
                     xq, x_scale, wq, w_scale, bias, y, m, n, k);
  return hipGetLastError();
}

template <int YT>
hipError_t launch_yt(const int8_t* xq, const float* x_scale, const int8_t* wq,
                     const float* w_scale, const float* bias, void* y, int64_t m, int64_t n,
                     int64_t k, hipStream_t stream) {
  const int64_t big_tiles = ((m + 255) / 256) * ((n + 255) / 256);
  if (big_tiles >= 192)
    return launch_cfg<256, 256, 2, 4, YT>(xq, x_scale, wq, w_scale, bias, y, m, n, k, stream);
  return launch_cfg<128, 128, 2, 2, YT>(xq, x_scale, wq, w_scale, bias, y, m, n, k, stream);
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
