// moe_steps.hip — the mixture-of-experts steps on either side of the grouped GEMM (gfx950):
// top-k routing from router logits, and the routing-weighted combine of the down
// projection's rows.  (SiLU·mul is fused into the grouped gate/up GEMM's epilogue.)
//
// "Phase 5a: int8 weight-only quantization" (Summary) runs the grouped GEMM inside the
// mixture-of-experts block of deepseek-moe-16b; no page spells out the block's other steps,
// so these kernels follow the plainest reading: softmax over the routed experts' logits, the
// k largest kept (unrenormalized) as routing weights, lower expert index first on equal
// logits, the always-on shared experts appended with weight 1; each token's output is the
// weighted sum of its assignments' rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace i8ql {
namespace {

constexpr int kRouteMaxPerLane = 4;  // logits held per lane: up to 256 routed experts

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Wavefront reductions with DPP moves (a few cycles each, instead of a round trip through
// the LDS crossbar per step): combine within pairs and quads, mirror within 8 and 16 lanes
// (every lane then holds its row of 16), then lane 15 of each row into rows 1 and 3 and lane
// 31 into rows 2 and 3.  Lanes those two moves do not write get their own value back (for a
// sum they double; only lane 63 is read): lane 63 ends with the result over all 64 lanes,
// which readlane broadcasts.
template <class Op>
__device__ __forceinline__ int wave_reduce(int v, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x141, 0xf, 0xf, false));  // row_half_mirror
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x140, 0xf, 0xf, false));  // row_mirror
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xa, 0xf, false));  // row_bcast15
  v = op(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xc, 0xf, false));  // row_bcast31
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_fmax(float f) {
  return __int_as_float(wave_reduce(__float_as_int(f), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }));
}

__device__ __forceinline__ float wave_fsum(float f) {
  return __int_as_float(wave_reduce(__float_as_int(f), [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }));
}

__device__ __forceinline__ int wave_imin(int v) {
  return wave_reduce(v, [](int a, int b) { return min(a, b); });
}

// One wavefront per token, four tokens per workgroup.  Lane l holds logits l, l + 64, ...;
// the k_routed picks are k_routed rounds of a wavefront arg-max over the lanes' best untaken
// candidates (the largest value, then the lowest index holding it), so the order of the
// slots is the selection order.  Lane s keeps slot s's id and weight and the wavefront
// stores all slots at once.
template <bool BF16>
__global__ __launch_bounds__(256) void moe_route_kernel(const void* __restrict__ logits,
                                                        int64_t t, int e_routed, int k_routed,
                                                        int n_shared, int32_t* __restrict__ ids,
                                                        float* __restrict__ weights) {
  const int lane = threadIdx.x % 64;
  const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + threadIdx.x / 64;
  if (tok >= t) return;  // whole wavefronts only: no barrier below
  float v[kRouteMaxPerLane];
  bool live[kRouteMaxPerLane];
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i) {
    const int j = lane + 64 * i;
    live[i] = j < e_routed;
    const int64_t off = tok * e_routed + (live[i] ? j : 0);
    if constexpr (BF16)
      v[i] = bf16_bits_to_f32(static_cast<const uint16_t*>(logits)[off]);
    else
      v[i] = static_cast<const float*>(logits)[off];
  }
  // softmax denominator over the routed experts, relative to the largest logit
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i)
    if (live[i]) mx = fmaxf(mx, v[i]);
  mx = wave_fmax(mx);
  float den = 0.0f;
#pragma unroll
  for (int i = 0; i < kRouteMaxPerLane; ++i)
    if (live[i]) den += expf(v[i] - mx);
  den = wave_fsum(den);

  int my_id = -1;
  float my_w = 0.0f;
  for (int s = 0; s < k_routed; ++s) {
    // this lane's best untaken logit (its indices ascend with i: the first of equal ones)
    float lv = -INFINITY;
    int li = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i)
      if (live[i] && (v[i] > lv || li == 0x7fffffff)) {
        lv = v[i];
        li = lane + 64 * i;
      }
    const float bv = wave_fmax(lv);
    const int bi = wave_imin(lv == bv ? li : 0x7fffffff);
    // every lane now holds the pick; its owner retires it
#pragma unroll
    for (int i = 0; i < kRouteMaxPerLane; ++i)
      if (lane + 64 * i == bi) live[i] = false;
    if (lane == s) {
      my_id = bi;
      my_w = expf(bv - mx) / den;
    }
  }
  if (lane >= k_routed && lane < k_routed + n_shared) {
    my_id = e_routed + (lane - k_routed);
    my_w = 1.0f;
  }
  const int kk = k_routed + n_shared;
  if (lane < kk) {
    ids[tok * kk + lane] = my_id;
    weights[tok * kk + lane] = my_w;
  }
}

// y[i, c] = sum_j w[i, j] * d[i * topk + j, c], float32 in slot order.  Workgroup (token,
// chunk of 256 * VEC channels); VEC = 8 reads 16 bytes of bf16 (or two of float32) per row.
template <int VEC, int DT, int YT>
__global__ __launch_bounds__(256) void moe_combine_kernel(const void* __restrict__ d,
                                                          const float* __restrict__ w,
                                                          int64_t topk, int64_t n,
                                                          void* __restrict__ y) {
  const int64_t tok = blockIdx.x;
  const int64_t c0 = (static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x) * VEC;
  if (c0 >= n) return;
  float acc[VEC];
#pragma unroll
  for (int u = 0; u < VEC; ++u) acc[u] = 0.0f;
  for (int64_t j = 0; j < topk; ++j) {
    const float wj = w[tok * topk + j];
    const int64_t row = (tok * topk + j) * n + c0;
    if constexpr (DT == I8QL_BF16) {
      if constexpr (VEC == 8) {
        const uint4 p = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(d) + row);
        const uint32_t q[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc[2 * u] += wj * __uint_as_float(q[u] << 16);
          acc[2 * u + 1] += wj * __uint_as_float(q[u] & 0xffff0000u);
        }
      } else {
        acc[0] += wj * bf16_bits_to_f32(static_cast<const uint16_t*>(d)[row]);
      }
    } else {
      if constexpr (VEC == 8) {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(d) + row);
        const float4 b =
            *reinterpret_cast<const float4*>(static_cast<const float*>(d) + row + 4);
        acc[0] += wj * a.x;
        acc[1] += wj * a.y;
        acc[2] += wj * a.z;
        acc[3] += wj * a.w;
        acc[4] += wj * b.x;
        acc[5] += wj * b.y;
        acc[6] += wj * b.z;
        acc[7] += wj * b.w;
      } else {
        acc[0] += wj * static_cast<const float*>(d)[row];
      }
    }
  }
  const int64_t out = tok * n + c0;
  if constexpr (YT == I8QL_BF16) {
    if constexpr (VEC == 8) {
      uint4 p;
      p.x = f32_to_bf16_bits(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[1])) << 16);
      p.y = f32_to_bf16_bits(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[3])) << 16);
      p.z = f32_to_bf16_bits(acc[4]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[5])) << 16);
      p.w = f32_to_bf16_bits(acc[6]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[7])) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + out) = p;
    } else {
      static_cast<uint16_t*>(y)[out] = f32_to_bf16_bits(acc[0]);
    }
  } else {
    if constexpr (VEC == 8) {
      float* yo = static_cast<float*>(y) + out;
      *reinterpret_cast<float4*>(yo) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(yo + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
      static_cast<float*>(y)[out] = acc[0];
    }
  }
}

template <int VEC, int DT>
hipError_t combine_yt(const void* d, const float* w, int64_t t, int64_t topk, int64_t n,
                      void* y, i8ql_dtype y_dtype, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(t), static_cast<unsigned>((n + 256 * VEC - 1) / (256 * VEC)));
  if (y_dtype == I8QL_F32)
    hipLaunchKernelGGL((moe_combine_kernel<VEC, DT, I8QL_F32>), grid, dim3(256), 0, stream, d,
                       w, topk, n, y);
  else
    hipLaunchKernelGGL((moe_combine_kernel<VEC, DT, I8QL_BF16>), grid, dim3(256), 0, stream, d,
                       w, topk, n, y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_route_topk(const void* logits, i8ql_dtype dtype, int64_t t,
                                 int64_t e_routed, int64_t k_routed, int64_t n_shared,
                                 int32_t* ids, float* weights, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((t + 3) / 4));
  if (dtype == I8QL_BF16)
    hipLaunchKernelGGL(moe_route_kernel<true>, grid, dim3(256), 0, stream, logits, t,
                       static_cast<int>(e_routed), static_cast<int>(k_routed),
                       static_cast<int>(n_shared), ids, weights);
  else
    hipLaunchKernelGGL(moe_route_kernel<false>, grid, dim3(256), 0, stream, logits, t,
                       static_cast<int>(e_routed), static_cast<int>(k_routed),
                       static_cast<int>(n_shared), ids, weights);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void* d, i8ql_dtype d_dtype, const float* weights,
                              int64_t t, int64_t topk, int64_t n, void* y, i8ql_dtype y_dtype,
                              hipStream_t stream) {
  // whole 16-byte row chunks of both operands: eight channels per thread
  const int es = d_dtype == I8QL_F32 ? 4 : 2;
  const bool vec = n % 8 == 0 && reinterpret_cast<uintptr_t>(d) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(y) % 16 == 0 && (n * es) % 16 == 0;
  if (d_dtype == I8QL_F32)
    return vec ? combine_yt<8, I8QL_F32>(d, weights, t, topk, n, y, y_dtype, stream)
               : combine_yt<1, I8QL_F32>(d, weights, t, topk, n, y, y_dtype, stream);
  return vec ? combine_yt<8, I8QL_BF16>(d, weights, t, topk, n, y, y_dtype, stream)
             : combine_yt<1, I8QL_BF16>(d, weights, t, topk, n, y, y_dtype, stream);
}

}  // namespace i8ql
