// quantize_rows.hip — symmetric absmax int8 quantization of the rows of a matrix (gfx950).
//
// One kernel serves both quantizers: per-output-channel weights and dynamic per-token
// activations apply the same rule to every row ("Day 6 — Quantize It Yourself", The
// mechanism, block 1: q = clamp(round(w / s)), s = absmax / largest code; "Phase 5a: int8
// weight-only quantization", Summary: float32 arithmetic and an all-zero-channel guard).
//
// Work layout: one 64-lane wavefront per row, four rows per 256-thread workgroup, or, for
// fewer than 1024 rows or rows of more than 768 chunks, a whole workgroup per row.  Pass 1
// streams the row with 16-byte loads (kept in registers when the row fits, up to 24 KiB per
// wavefront), reduces |a| to
// the row maximum with cross-lane shuffles (and LDS across wavefronts); pass 2 divides,
// rounds and packs 4 or 8 codes per store.  The row is read from HBM once; the op is HBM-bound
// (2 + 1 bytes per bf16 element).
//
// Arithmetic (identical for every dtype): the input is widened exactly to float32;
// s = amax / 127 is a correctly rounded float32 division; s == 0 stores scale 1 and zero
// codes; otherwise each code is rint(a / s) (the correctly rounded float32 quotient, then
// round half to even via v_rndne_f32) clamped to [-127, 127].  The quotient comes from the
// reciprocal and one FMA correction (see quotient_fma), which yields exactly the correctly
// rounded quotient at a third of the instructions of a full division.  The file must not be
// built with fast-math.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace i8ql {
namespace {

constexpr int kWave = 64;
constexpr int kRowsPerBlock = 4;
constexpr int kCacheChunks = 24;  // 16-byte chunks per lane kept in registers (24 KiB rows)
constexpr int64_t kSplitRowsBelow = 1024;  // fewer rows: four wavefronts per row

template <int DT>
struct Fmt;
template <>
struct Fmt<I8QL_F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
};
template <>
struct Fmt<I8QL_BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
};
template <>
struct Fmt<I8QL_F16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
};

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
  _Float16 v;
  uint16_t b = static_cast<uint16_t>(h);
  __builtin_memcpy(&v, &b, 2);
  return static_cast<float>(v);
}

// Widen one 16-byte chunk to float32 (exact for every input format).
template <int DT>
__device__ __forceinline__ void widen_chunk(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (DT == I8QL_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (DT == I8QL_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = half_bits_to_f32(w[i] & 0xffffu);
      f[2 * i + 1] = half_bits_to_f32(w[i] >> 16);
    }
  }
}

template <int DT>
__device__ __forceinline__ float widen_one(const void* base, int64_t i) {
  if constexpr (DT == I8QL_F32) {
    return static_cast<const float*>(base)[i];
  } else if constexpr (DT == I8QL_BF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
  } else {
    return half_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  }
}

// Maximum of a non-negative float over the 64 lanes, returned in every lane.  Non-negative
// floats order like their bit patterns, so the reduction runs on integers with DPP moves
// (swap within pairs and quads, mirror within 8 and 16 lanes, then broadcast lane 15 of each
// row into the next row and lane 31 into the upper half); lane 63 ends with the maximum.
__device__ __forceinline__ float wave_max(float f) {
  int v = __float_as_int(f);
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));  // row_mirror
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));  // row_bcast15
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));  // row_bcast31
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

// RN(a / s) from y = RN(1 / s) and fused multiply-adds: q0 = RN(a * y) is within one ulp of
// a / s, the remainder r = a - s * q0 is then exactly representable (one FMA computes it
// without rounding), and RN(q0 + r * y) is the correctly rounded quotient RN(a / s) whenever
// no intermediate underflows (Markstein's theorem for division with an FMA, P. Markstein,
// IBM J. Res. Dev. 34(1), 1990; also the division chapter of Muller et al., Handbook of
// Floating-Point Arithmetic).  The remainder can only underflow for |a| below about 2^-102.
// The caller takes this path only for s >= 2^-64: an element whose code can be nonzero has
// |a| >= s / 2 >= 2^-65, and a smaller |a| has a quotient below 1/2 in magnitude, which
// rounds to code 0 whatever its last bits.
__device__ __forceinline__ float quotient_fma(float a, float s, float y) {
  const float q0 = a * y;
  const float r = __builtin_fmaf(-s, q0, a);
  return __builtin_fmaf(r, y, q0);
}

// The code of one element from a quotient: ties-to-even, clamp.
__device__ __forceinline__ int code_from_quotient(float q) {
  return static_cast<int>(__builtin_amdgcn_fmed3f(rintf(q), -127.0f, 127.0f));
}

// The code of one element: correctly rounded float32 quotient, ties-to-even, clamp.
__device__ __forceinline__ int code_of(float a, float s) {
  float t = rintf(a / s);
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return static_cast<int>(t);
}

__device__ __forceinline__ float chunk_absmax(const float* f, int n, float m) {
  for (int i = 0; i < n; ++i) m = fmaxf(m, fabsf(f[i]));
  return m;
}

// Vector path: row bytes are a multiple of 16 and the base is 16-byte aligned.  W wavefronts
// share a row (W = 4 when there are few rows, so that short launches still fill the CUs;
// their maxima meet in LDS); a workgroup holds 4 / W rows.  Every lane loads all of its
// chunks before it uses one: loads past the row's end re-read its last chunk (harmless to
// the maximum, never stored), so they are unconditional and all in flight together.
// The rows of workgroup `block` of one matrix (used by the single-matrix kernel and, per
// matrix, by the kernel that quantizes several in one launch).
template <int DT, int W>
__device__ __forceinline__ void vec_rows(const uint8_t* __restrict__ a, int64_t rows, int64_t k,
                                         int8_t* __restrict__ q, float* __restrict__ scale,
                                         int64_t block, float* wmax) {
  constexpr int E = Fmt<DT>::kPerChunk;
  constexpr int T = kWave * W;  // threads per row
  const int t = threadIdx.x % T;
  const int slot = threadIdx.x / T;  // row within the workgroup
  const int64_t row = block * (kRowsPerBlock / W) + slot;
  const bool live = row < rows;  // whole rows only; a dead row still joins the barrier
  const int64_t rr = live ? row : rows - 1;
  const int64_t chunks = k / E;
  const uint4* src = reinterpret_cast<const uint4*>(a + rr * k * Fmt<DT>::kBytes);
  int8_t* dst = q + rr * k;
  const bool cached = chunks <= static_cast<int64_t>(kCacheChunks) * T;

  uint4 cache[kCacheChunks];
  float amax = 0.0f;
  float f[E];
  if (cached) {
#pragma unroll
    for (int i = 0; i < kCacheChunks; ++i) {
      const int64_t c = t + static_cast<int64_t>(i) * T;
      if (static_cast<int64_t>(i) * T < chunks) cache[i] = src[c < chunks ? c : chunks - 1];
    }
#pragma unroll
    for (int i = 0; i < kCacheChunks; ++i) {
      if (static_cast<int64_t>(i) * T < chunks) {
        widen_chunk<DT>(cache[i], f);
        amax = chunk_absmax(f, E, amax);
      }
    }
  } else {
    for (int64_t c = t; c < chunks; c += T) {
      widen_chunk<DT>(src[c], f);
      amax = chunk_absmax(f, E, amax);
    }
  }
  amax = wave_max(amax);
  if constexpr (W > 1) {
    if (threadIdx.x % kWave == 0) wmax[threadIdx.x / kWave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < W; ++w) amax = fmaxf(amax, wmax[slot * W + w]);
  }
  if (!live) return;
  const float s = amax / 127.0f;

  if (s == 0.0f) {  // all-zero channel: scale 1, codes 0
    for (int64_t j = t * 4; j < k; j += T * 4)
      *reinterpret_cast<uint32_t*>(dst + j) = 0u;  // k % 4 == 0 on this path
    if (t == 0) scale[row] = 1.0f;
    return;
  }

  // Pass 2 with the quotients from the reciprocal (scales of 2^-64 and up: every row of
  // practical data) or from full divisions (smaller scales); one branch per row.
  auto emit_all = [&](auto code) {
    auto emit = [&](const uint4 v, int64_t c) {
      widen_chunk<DT>(v, f);
      uint32_t packed[E / 4];
#pragma unroll
      for (int g = 0; g < E / 4; ++g) {
        uint32_t p = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          p |= (static_cast<uint32_t>(code(f[4 * g + b])) & 0xffu) << (8 * b);
        packed[g] = p;
      }
      if constexpr (E == 4) {
        *reinterpret_cast<uint32_t*>(dst + c * 4) = packed[0];
      } else {
        *reinterpret_cast<uint2*>(dst + c * 8) = make_uint2(packed[0], packed[1]);
      }
    };
    if (cached) {
#pragma unroll
      for (int i = 0; i < kCacheChunks; ++i) {
        const int64_t c = t + static_cast<int64_t>(i) * T;
        if (c < chunks) emit(cache[i], c);
      }
    } else {
      for (int64_t c = t; c < chunks; c += T) emit(src[c], c);
    }
  };
  if (s >= 0x1p-64f) {
    const float y = 1.0f / s;  // RN(1 / s)
    emit_all([&](float a) { return code_from_quotient(quotient_fma(a, s, y)); });
  } else {
    emit_all([&](float a) { return code_of(a, s); });
  }
  if (t == 0) scale[row] = s;
}

template <int DT, int W>
__global__ __launch_bounds__(kWave* kRowsPerBlock) void quantize_rows_vec_kernel(
    const uint8_t* __restrict__ a, int64_t rows, int64_t k, int8_t* __restrict__ q,
    float* __restrict__ scale) {
  __shared__ float wmax[kRowsPerBlock];
  vec_rows<DT, W>(a, rows, k, q, scale, blockIdx.x, wmax);
}

// Several matrices in one launch: matrix j owns workgroups [first[j], first[j + 1]) and is
// quantized exactly as by itself (the same rows per workgroup and wavefronts per row).
struct MultiJobs {
  const uint8_t* a[I8QL_QUANT_MAX_JOBS];
  int8_t* q[I8QL_QUANT_MAX_JOBS];
  float* scale[I8QL_QUANT_MAX_JOBS];
  int64_t rows[I8QL_QUANT_MAX_JOBS];
  int64_t k[I8QL_QUANT_MAX_JOBS];
  int64_t first[I8QL_QUANT_MAX_JOBS + 1];
  int w4[I8QL_QUANT_MAX_JOBS];  // 1: four wavefronts per row
  int count;
};

template <int DT>
__global__ __launch_bounds__(kWave* kRowsPerBlock) void quantize_rows_multi_kernel(MultiJobs jobs) {
  __shared__ float wmax[kRowsPerBlock];
  const int64_t b = blockIdx.x;
  int j = 0;
  while (j + 1 < jobs.count && b >= jobs.first[j + 1]) ++j;
  const int64_t block = b - jobs.first[j];
  if (jobs.w4[j])
    vec_rows<DT, 4>(jobs.a[j], jobs.rows[j], jobs.k[j], jobs.q[j], jobs.scale[j], block, wmax);
  else
    vec_rows<DT, 1>(jobs.a[j], jobs.rows[j], jobs.k[j], jobs.q[j], jobs.scale[j], block, wmax);
}

// Scalar path: any k and any element-aligned base.
template <int DT>
__global__ __launch_bounds__(kWave* kRowsPerBlock) void quantize_rows_scalar_kernel(
    const void* __restrict__ a, int64_t rows, int64_t k, int8_t* __restrict__ q,
    float* __restrict__ scale) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= rows) return;
  const int64_t base = row * k;
  float amax = 0.0f;
  for (int64_t j = lane; j < k; j += kWave) amax = fmaxf(amax, fabsf(widen_one<DT>(a, base + j)));
  amax = wave_max(amax);
  const float s = amax / 127.0f;
  if (s == 0.0f) {
    for (int64_t j = lane; j < k; j += kWave) q[base + j] = 0;
    if (lane == 0) scale[row] = 1.0f;
    return;
  }
  for (int64_t j = lane; j < k; j += kWave)
    q[base + j] = static_cast<int8_t>(code_of(widen_one<DT>(a, base + j), s));
  if (lane == 0) scale[row] = s;
}

// four wavefronts per row when one per row would leave the CUs short of wavefronts (fewer
// than kSplitRowsBelow rows in the launch: `launch_rows`), or give each lane more than 12
// chunks
template <int DT>
bool four_waves_per_row(int64_t rows, int64_t k, int64_t launch_rows) {
  const int64_t chunks = k / Fmt<DT>::kPerChunk;
  return (launch_rows < kSplitRowsBelow || chunks > 12 * kWave) && rows <= INT32_MAX;
}

template <int DT>
hipError_t launch_dt(const void* a, int64_t rows, int64_t k, int8_t* q, float* scale,
                     hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  const dim3 block(kWave * kRowsPerBlock);
  const bool vec = (k * Fmt<DT>::kBytes) % 16 == 0 &&
                   (reinterpret_cast<uintptr_t>(a) % 16) == 0 &&
                   (reinterpret_cast<uintptr_t>(q) % 8) == 0;
  if (vec && four_waves_per_row<DT>(rows, k, rows)) {
    const dim3 grid4(static_cast<unsigned>(rows));
    hipLaunchKernelGGL((quantize_rows_vec_kernel<DT, 4>), grid4, block, 0, stream,
                       static_cast<const uint8_t*>(a), rows, k, q, scale);
  } else if (vec) {
    hipLaunchKernelGGL((quantize_rows_vec_kernel<DT, 1>), grid, block, 0, stream,
                       static_cast<const uint8_t*>(a), rows, k, q, scale);
  } else {
    hipLaunchKernelGGL(quantize_rows_scalar_kernel<DT>, grid, block, 0, stream, a, rows, k, q,
                       scale);
  }
  return hipGetLastError();
}

// ---- one scale per group of 128 input channels ------------------------------------------
// "Day 6 — Quantize It Yourself" (The mechanism, block 1): finer than one scale per output
// channel, each run of 128 consecutive input channels of a row gets its own.  The rule per group is
// the row rule above.  Since k is a multiple of 128, the [n, k] matrix is a plain sequence
// of groups and the [n, k / 128] scale matrix lists them in the same order: thread i takes
// elements 8i .. 8i + 7, sixteen consecutive lanes (one DPP row) hold one group, and the
// group maximum is a four-step DPP reduction inside that row.
template <int DT>
__global__ __launch_bounds__(256) void quantize_groups128_kernel(const uint8_t* __restrict__ a,
                                                                 int64_t total,
                                                                 int8_t* __restrict__ q,
                                                                 float* __restrict__ scale) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  const bool live = e < total;  // whole groups: a group's 16 lanes are all live or all not
  const int64_t ee = live ? e : 0;
  float f[8];
  if constexpr (DT == I8QL_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(a + ee * 4);
    widen_chunk<DT>(p[0], f);
    widen_chunk<DT>(p[1], f + 4);
  } else {
    widen_chunk<DT>(*reinterpret_cast<const uint4*>(a + ee * 2), f);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  // group maximum: non-negative floats order like their bit patterns
  int v = __float_as_int(amax);
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));  // row_mirror
  amax = __int_as_float(v);
  if (!live) return;
  const float s = amax / 127.0f;
  int c[8];
  if (s == 0.0f) {  // all-zero group: scale 1, codes 0
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = 0;
  } else if (s >= 0x1p-64f) {
    const float y = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = code_from_quotient(quotient_fma(f[i], s, y));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = code_of(f[i], s);
  }
  uint2 packed;
  packed.x = (c[0] & 0xff) | ((c[1] & 0xff) << 8) | ((c[2] & 0xff) << 16) |
             (static_cast<uint32_t>(c[3] & 0xff) << 24);
  packed.y = (c[4] & 0xff) | ((c[5] & 0xff) << 8) | ((c[6] & 0xff) << 16) |
             (static_cast<uint32_t>(c[7] & 0xff) << 24);
  *reinterpret_cast<uint2*>(q + e) = packed;
  if (threadIdx.x % 16 == 0) scale[e / 128] = s == 0.0f ? 1.0f : s;
}

// ---- RMS norm fused with the per-token quantization ----------------------------------
// The producer of a decoder layer's q/k/v and gate/up inputs is an RMS norm of the residual
// stream.  Quantizing inside it writes the int8 codes (1 byte per element) where a separate
// quantizer would first write the bf16 norm output and read it back (2 + 2 bytes): dynamic
// per-token activation quantization ("feat(quantization): support compressed-tensors W8A8
// and mixed modules", Design and Supported Execution Scheme) then costs no extra pass over
// the activations ("Day 6 — Quantize It Yourself", Reading-share post, fact 2, on the work
// it adds to the forward pass).  The norm itself is not on the pages; the reading:
//   u = x, or u = bf16(x + residual) (one float32 addition), also stored as the new residual;
//   S = sum of u^2 in float64 (each square is exact, so the sum carries about 2^-50 relative
//   error whatever its order and rounds to the same float32 mean as any other order except
//   within that distance of a rounding midpoint);  v = fl32(S / k);
//   r = fl32(1 / fl32(sqrt(fl32(v + eps))));   h = bf16(fl32(fl32(u * r) * gamma));
// then the row rule above on h, which is bitwise what quantize_rows gives for the bf16 norm
// output.  Layout as the row quantizer: W wavefronts per row, every chunk of the row (and of
// gamma, and of the residual) loaded before any is used and kept in registers, rows of up to
// kNormChunks * 64 * W chunks of 8 elements.
constexpr int kNormChunks = 12;

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {  // finite f
  uint32_t b = __float_as_uint(f);
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  return bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
}

// Sum over the 64 lanes in float64 (a butterfly: every lane ends with the same value).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// The row rule on a bf16 row held in registers (u[i]: chunk t + i * 64 W of the row, for the
// i with i * 64 W < chunks; chunks past the row end repeat its last chunk), given this lane's
// share of the row maximum: the maximum over the W wavefronts of the row, then the codes
// (8 per chunk, one 8-byte store each) and the scale, exactly as the row quantizer.
template <int W>
__device__ __forceinline__ void quantize_held_row(const uint4 (&u)[kNormChunks], float amax,
                                                  int64_t chunks, int t, int slot, bool live,
                                                  int64_t row, int64_t row_base,
                                                  int8_t* __restrict__ q,
                                                  float* __restrict__ scale, float* wmax) {
  constexpr int T = kWave * W;
  amax = wave_max(amax);
  if constexpr (W > 1) {
    if (threadIdx.x % kWave == 0) wmax[threadIdx.x / kWave] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < W; ++w) amax = fmaxf(amax, wmax[slot * W + w]);
  }
  if (!live) return;
  const float s = amax / 127.0f;
  int8_t* dst = q + row_base;
  auto emit_all = [&](auto code) {
#pragma unroll
    for (int i = 0; i < kNormChunks; ++i) {
      const int64_t c0 = t + static_cast<int64_t>(i) * T;
      if (static_cast<int64_t>(i) * T < chunks && c0 < chunks) {
        float f[8];
        widen_chunk<I8QL_BF16>(u[i], f);
        uint32_t p[2];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          uint32_t w = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            w |= (static_cast<uint32_t>(code(f[4 * g2 + b])) & 0xffu) << (8 * b);
          p[g2] = w;
        }
        *reinterpret_cast<uint2*>(dst + c0 * 8) = make_uint2(p[0], p[1]);
      }
    }
  };
  if (s == 0.0f) {
    emit_all([](float) { return 0; });
    if (t == 0) scale[row] = 1.0f;
    return;
  }
  if (s >= 0x1p-64f) {
    const float y = 1.0f / s;
    emit_all([&](float a) { return code_from_quotient(quotient_fma(a, s, y)); });
  } else {
    emit_all([&](float a) { return code_of(a, s); });
  }
  if (t == 0) scale[row] = s;
}

template <int W, bool QUANT, bool RES>
__global__ __launch_bounds__(kWave* kRowsPerBlock) void rmsnorm_rows_kernel(
    const uint4* __restrict__ x, uint4* __restrict__ res, const uint4* __restrict__ gamma,
    float eps, int64_t rows, int64_t k, int8_t* __restrict__ q, float* __restrict__ scale,
    uint4* __restrict__ h_out) {
  constexpr int T = kWave * W;  // threads per row
  __shared__ double wsum[kRowsPerBlock];
  __shared__ float wmax[kRowsPerBlock];
  const int t = threadIdx.x % T;
  const int slot = threadIdx.x / T;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kRowsPerBlock / W) + slot;
  const bool live = row < rows;  // a dead row still joins the barriers
  const int64_t rr = live ? row : rows - 1;
  const int64_t chunks = k / 8;
  const int64_t base = rr * chunks;

  // every load in flight first (chunks past the row end re-read its last chunk: never used)
  uint4 u[kNormChunks], gm[kNormChunks], rv[kNormChunks];
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    if (static_cast<int64_t>(i) * T < chunks) {
      const int64_t c0 = t + static_cast<int64_t>(i) * T;
      const int64_t c = c0 < chunks ? c0 : chunks - 1;
      u[i] = x[base + c];
      if constexpr (RES) rv[i] = res[base + c];
      gm[i] = gamma[c];
    }
  }
  // residual add (stored back as the new residual) and the float64 sum of squares
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    if (static_cast<int64_t>(i) * T < chunks) {
      const int64_t c0 = t + static_cast<int64_t>(i) * T;
      float f[8];
      widen_chunk<I8QL_BF16>(u[i], f);
      if constexpr (RES) {
        float r[8];
        widen_chunk<I8QL_BF16>(rv[i], r);
        u[i] = make_uint4(bf16_pack(f[0] + r[0], f[1] + r[1]), bf16_pack(f[2] + r[2], f[3] + r[3]),
                          bf16_pack(f[4] + r[4], f[5] + r[5]), bf16_pack(f[6] + r[6], f[7] + r[7]));
        widen_chunk<I8QL_BF16>(u[i], f);
        if (live && c0 < chunks) res[base + c0] = u[i];
      }
      if (c0 < chunks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double d = static_cast<double>(f[e]);
          ss += d * d;  // exact square; fused or not, the same sum
        }
      }
    }
  }
  ss = wave_sum_f64(ss);
  if constexpr (W > 1) {
    if (threadIdx.x % kWave == 0) wsum[threadIdx.x / kWave] = ss;
    __syncthreads();
    ss = wsum[slot * W];
#pragma unroll
    for (int w = 1; w < W; ++w) ss += wsum[slot * W + w];
  }
  const float v = static_cast<float>(ss / static_cast<double>(k));
  const float rs = 1.0f / sqrtf(v + eps);

  // h = bf16((u * r) * gamma), kept in u; its row maximum
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    if (static_cast<int64_t>(i) * T < chunks) {
      float f[8], g[8];
      widen_chunk<I8QL_BF16>(u[i], f);
      widen_chunk<I8QL_BF16>(gm[i], g);
      float hv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = (f[e] * rs) * g[e];
      u[i] = make_uint4(bf16_pack(hv[0], hv[1]), bf16_pack(hv[2], hv[3]),
                        bf16_pack(hv[4], hv[5]), bf16_pack(hv[6], hv[7]));
      if constexpr (QUANT) {
        widen_chunk<I8QL_BF16>(u[i], f);  // (re-read clamped chunks too: harmless to the max)
        amax = chunk_absmax(f, 8, amax);
      } else {
        const int64_t c0 = t + static_cast<int64_t>(i) * T;
        if (live && c0 < chunks) h_out[base + c0] = u[i];
      }
    }
  }
  if constexpr (QUANT)
    quantize_held_row<W>(u, amax, chunks, t, slot, live, row, rr * k, q, scale, wmax);
}

template <bool QUANT, bool RES>
hipError_t launch_rmsnorm_t(const void* x, void* res, const void* gamma, float eps, int64_t rows,
                            int64_t k, int8_t* q, float* scale, void* h, hipStream_t stream) {
  const dim3 block(kWave * kRowsPerBlock);
  const auto* xs = static_cast<const uint4*>(x);
  auto* rs = static_cast<uint4*>(res);
  const auto* gs = static_cast<const uint4*>(gamma);
  auto* hs = static_cast<uint4*>(h);
  if (four_waves_per_row<I8QL_BF16>(rows, k, rows)) {
    hipLaunchKernelGGL((rmsnorm_rows_kernel<4, QUANT, RES>), dim3(static_cast<unsigned>(rows)),
                       block, 0, stream, xs, rs, gs, eps, rows, k, q, scale, hs);
  } else {
    hipLaunchKernelGGL((rmsnorm_rows_kernel<1, QUANT, RES>),
                       dim3(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                       block, 0, stream, xs, rs, gs, eps, rows, k, q, scale, hs);
  }
  return hipGetLastError();
}

// ---- SiLU·mul fused with the per-token quantization ------------------------------------
// The down projection's input is silu(gate) * up of the gate/up projection's output, one row
// per token: gu [m, 2 n] bf16 with the gate values in columns [0, n) and the up values in
// [n, 2 n) (one GEMM over the stacked gate and up weights).  Quantizing while the activation
// is formed writes the int8 codes (1 byte per element) instead of the bf16 activation that a
// separate quantizer would read back (2 + 2 bytes).  Per element, in float32:
//   h = g * rcp(1 + exp(-g)) * u,  then bf16 (ties to even),
// the exponential within about 2^-19.5 (relative) and the reciprocal within an ulp, so h
// lies within about 2^-19 of the exact value; elements that float32 cannot
// resolve (g < -80, where e^-g approaches the float range, and nonzero |h| < 2^-120, where
// the product leaves the normal range) are formed in float64 instead.  The rounding to bf16
// then differs from that of the exact value only for values within that distance of the
// halfway point between two bf16 values.  Layout as the RMS norm above: W wavefronts per row,
// every chunk of the row's gate and up halves loaded before any is used and h kept in
// registers for the row rule.
__device__ __forceinline__ float silu_mul_one(float g, float u) {
  // e^-g: for g >= -16 as 2^(-g log2 e) with the hardware exponential (the rounding of the
  // product moves the result by at most |g| 2^-24 relative, the exponential by about an
  // ulp; for g > 16 the term vanishes next to 1 anyway), below -16 the accurate expf (one
  // branch per wavefront, taken only when some lane needs it)
  float e;
  if (__builtin_amdgcn_ballot_w64(g < -16.0f) == 0) {
    e = __expf(-g);
  } else {
    e = g >= -16.0f ? __expf(-g) : expf(-g);
  }
  float h = g * __builtin_amdgcn_rcpf(1.0f + e) * u;
  if (g < -80.0f || (h != 0.0f && fabsf(h) < 0x1p-120f)) {
    const double gd = g, ud = u;
    h = static_cast<float>(gd / (1.0 + exp(-gd)) * ud);
  }
  return h;
}

template <int W, bool QUANT>
__global__ __launch_bounds__(kWave* kRowsPerBlock) void silu_mul_rows_kernel(
    const uint4* __restrict__ gu, int64_t rows, int64_t n, int8_t* __restrict__ q,
    float* __restrict__ scale, uint4* __restrict__ h_out) {
  constexpr int T = kWave * W;  // threads per row
  __shared__ float wmax[kRowsPerBlock];
  const int t = threadIdx.x % T;
  const int slot = threadIdx.x / T;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kRowsPerBlock / W) + slot;
  const bool live = row < rows;  // a dead row still joins the barriers
  const int64_t rr = live ? row : rows - 1;
  const int64_t chunks = n / 8;  // of each half
  const uint4* gate = gu + rr * 2 * chunks;
  const uint4* up = gate + chunks;

  uint4 u[kNormChunks], ug[kNormChunks];
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    if (static_cast<int64_t>(i) * T < chunks) {
      const int64_t c0 = t + static_cast<int64_t>(i) * T;
      const int64_t c = c0 < chunks ? c0 : chunks - 1;
      u[i] = gate[c];
      ug[i] = up[c];
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kNormChunks; ++i) {
    if (static_cast<int64_t>(i) * T < chunks) {
      float g[8], v[8], hv[8];
      widen_chunk<I8QL_BF16>(u[i], g);
      widen_chunk<I8QL_BF16>(ug[i], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = silu_mul_one(g[e], v[e]);
      u[i] = make_uint4(bf16_pack(hv[0], hv[1]), bf16_pack(hv[2], hv[3]),
                        bf16_pack(hv[4], hv[5]), bf16_pack(hv[6], hv[7]));
      if constexpr (QUANT) {
        widen_chunk<I8QL_BF16>(u[i], hv);
        amax = chunk_absmax(hv, 8, amax);
      } else {
        const int64_t c0 = t + static_cast<int64_t>(i) * T;
        if (live && c0 < chunks) h_out[rr * chunks + c0] = u[i];
      }
    }
  }
  if constexpr (QUANT)
    quantize_held_row<W>(u, amax, chunks, t, slot, live, row, rr * n, q, scale, wmax);
}

template <bool QUANT>
hipError_t launch_silu_mul_t(const void* gu, int64_t rows, int64_t n, int8_t* q, float* scale,
                             void* h, hipStream_t stream) {
  const dim3 block(kWave * kRowsPerBlock);
  const auto* src = static_cast<const uint4*>(gu);
  auto* hs = static_cast<uint4*>(h);
  if (four_waves_per_row<I8QL_BF16>(rows, n, rows)) {
    hipLaunchKernelGGL((silu_mul_rows_kernel<4, QUANT>), dim3(static_cast<unsigned>(rows)),
                       block, 0, stream, src, rows, n, q, scale, hs);
  } else {
    hipLaunchKernelGGL((silu_mul_rows_kernel<1, QUANT>),
                       dim3(static_cast<unsigned>((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                       block, 0, stream, src, rows, n, q, scale, hs);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_groups128(const void* a, i8ql_dtype dtype, int64_t n, int64_t k,
                                     int8_t* q, float* scale, hipStream_t stream) {
  const int64_t total = n * k;
  const dim3 grid(static_cast<unsigned>((total / 8 + 255) / 256));
  const auto* src = static_cast<const uint8_t*>(a);
  switch (dtype) {
    case I8QL_F32:
      hipLaunchKernelGGL(quantize_groups128_kernel<I8QL_F32>, grid, dim3(256), 0, stream, src,
                         total, q, scale);
      break;
    case I8QL_BF16:
      hipLaunchKernelGGL(quantize_groups128_kernel<I8QL_BF16>, grid, dim3(256), 0, stream, src,
                         total, q, scale);
      break;
    case I8QL_F16:
      hipLaunchKernelGGL(quantize_groups128_kernel<I8QL_F16>, grid, dim3(256), 0, stream, src,
                         total, q, scale);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_multi_dt(const i8ql_quant_job* jobs, int count, hipStream_t stream) {
  MultiJobs mj = {};
  int64_t blocks = 0;
  int live = 0;
  // the matrices share the launch: whether one wavefront per row fills the CUs depends on
  // the rows of all of them (the four 512-token inputs of the dense 4B decoder layer: one
  // launch went from 11.1 to 8.5 us with this rule)
  int64_t launch_rows = 0;
  for (int i = 0; i < count; ++i) launch_rows += jobs[i].rows;
  for (int i = 0; i < count; ++i) {
    if (jobs[i].rows == 0) continue;  // nothing to quantize
    const bool w4 = four_waves_per_row<DT>(jobs[i].rows, jobs[i].k, launch_rows);
    mj.a[live] = static_cast<const uint8_t*>(jobs[i].x);
    mj.q[live] = jobs[i].q_out;
    mj.scale[live] = jobs[i].scale_out;
    mj.rows[live] = jobs[i].rows;
    mj.k[live] = jobs[i].k;
    mj.w4[live] = w4 ? 1 : 0;
    mj.first[live] = blocks;
    blocks += w4 ? jobs[i].rows : (jobs[i].rows + kRowsPerBlock - 1) / kRowsPerBlock;
    ++live;
  }
  if (live == 0) return hipSuccess;
  mj.first[live] = blocks;
  mj.count = live;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_rows_multi_kernel<DT>, dim3(static_cast<unsigned>(blocks)),
                     dim3(kWave * kRowsPerBlock), 0, stream, mj);
  return hipGetLastError();
}

hipError_t launch_quantize_rows_multi(const i8ql_quant_job* jobs, int count, i8ql_dtype dtype,
                                      hipStream_t stream) {
  switch (dtype) {
    case I8QL_F32: return launch_multi_dt<I8QL_F32>(jobs, count, stream);
    case I8QL_BF16: return launch_multi_dt<I8QL_BF16>(jobs, count, stream);
    case I8QL_F16: return launch_multi_dt<I8QL_F16>(jobs, count, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_rmsnorm(const void* x, void* residual, const void* gamma, float eps,
                         int64_t rows, int64_t k, int8_t* q, float* scale, void* h,
                         hipStream_t stream) {
  if (q) {
    return residual ? launch_rmsnorm_t<true, true>(x, residual, gamma, eps, rows, k, q, scale,
                                                   h, stream)
                    : launch_rmsnorm_t<true, false>(x, residual, gamma, eps, rows, k, q, scale,
                                                    h, stream);
  }
  return residual ? launch_rmsnorm_t<false, true>(x, residual, gamma, eps, rows, k, q, scale, h,
                                                  stream)
                  : launch_rmsnorm_t<false, false>(x, residual, gamma, eps, rows, k, q, scale,
                                                   h, stream);
}

hipError_t launch_silu_mul(const void* gu, int64_t rows, int64_t n, int8_t* q, float* scale,
                          void* h, hipStream_t stream) {
  return q ? launch_silu_mul_t<true>(gu, rows, n, q, scale, h, stream)
           : launch_silu_mul_t<false>(gu, rows, n, q, scale, h, stream);
}

hipError_t launch_quantize_rows(const void* a, i8ql_dtype dtype, int64_t rows, int64_t k,
                                int8_t* q, float* scale, hipStream_t stream) {
  switch (dtype) {
    case I8QL_F32: return launch_dt<I8QL_F32>(a, rows, k, q, scale, stream);
    case I8QL_BF16: return launch_dt<I8QL_BF16>(a, rows, k, q, scale, stream);
    case I8QL_F16: return launch_dt<I8QL_F16>(a, rows, k, q, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace i8ql
