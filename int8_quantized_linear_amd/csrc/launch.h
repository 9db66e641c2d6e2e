// launch.h — host-side launchers of the gfx950 kernels (internal to libi8ql).
//
// Each launcher assumes its arguments were validated by the C ABI layer (api.cpp): shapes
// non-negative and non-empty, dtypes supported, pointers non-NULL and aligned as the kernel
// requires.  Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "i8ql.h"

namespace i8ql {

// Raise kernel KERN's dynamic-LDS limit to at least `bytes` on the current device.  The
// attribute is set once per (kernel, device) and again only when a call needs more than was
// granted, so steady-state launches make no attribute call; concurrent first calls may both
// set it, which is harmless.
constexpr int kMaxDevices = 64;
template <auto KERN>
hipError_t allow_dynamic_lds(int bytes) {
  static std::atomic<int> granted[kMaxDevices];  // static storage: starts at zero
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool tracked = dev >= 0 && dev < kMaxDevices;
  if (tracked && granted[dev].load(std::memory_order_relaxed) >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(KERN),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && tracked) {
    int prev = granted[dev].load(std::memory_order_relaxed);
    while (prev < bytes && !granted[dev].compare_exchange_weak(prev, bytes)) {
    }
  }
  return e;
}

hipError_t launch_quantize_rows(const void* a, i8ql_dtype dtype, int64_t rows, int64_t k,
                                int8_t* q, float* scale, hipStream_t stream);

// RMS norm of bf16 rows (optional residual add, stored back) fused with the per-token int8
// quantization (q and scale non-NULL), or written as bf16 rows h (q NULL); validated:
// k % 8 == 0, k <= I8QL_NORM_MAX_K, 16-byte aligned rows.
hipError_t launch_rmsnorm(const void* x, void* residual, const void* gamma, float eps,
                         int64_t rows, int64_t k, int8_t* q, float* scale, void* h,
                         hipStream_t stream);

// SiLU·mul of a gate/up product gu [rows, 2n] bf16 (gate columns first) fused with the
// per-token int8 quantization (q and scale non-NULL), or written as bf16 rows h [rows, n]
// (q NULL); validated: n % 8 == 0, n <= I8QL_SILU_MAX_N, 16-byte aligned rows.
hipError_t launch_silu_mul(const void* gu, int64_t rows, int64_t n, int8_t* q, float* scale,
                          void* h, hipStream_t stream);

// Several matrices (validated for the vector path) in one launch.
hipError_t launch_quantize_rows_multi(const i8ql_quant_job* jobs, int count, i8ql_dtype dtype,
                                      hipStream_t stream);

// W8A8: plan (config, splits) = one of the I8QL_W8A8_NUM_CONFIGS tile configurations with
// k split across `splits` workgroups per tile (workspace ws of ws_bytes, zero counters), or
// config -1 for the plan the cost model chooses for this shape on the current device among
// those whose workspace fits in ws_bytes (none when ws is NULL).
hipError_t launch_w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                            const float* w_scale, const float* bias, void* y,
                            i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k, int config,
                            int splits, void* ws, int64_t ws_bytes, hipStream_t stream);

// launch_w8a8_gemm with the library's static scratch array (I8QL_W8A8_SCRATCH_BYTES per
// device) as the workspace: allocates nothing.
hipError_t launch_w8a8_gemm_noalloc(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                    const float* w_scale, const float* bias, void* y,
                                    i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                    int config, int splits, hipStream_t stream);

// Host only: the cost model's configuration with no split (w8a8_choose_config) or its plan
// within a workspace budget (w8a8_choose_plan), for `cus` compute units; the workspace a plan
// needs; whether a plan is valid for a shape; {tile rows, tile columns, k-groups, splittable}
// of a configuration.
int w8a8_choose_config(int64_t m, int64_t n, int64_t k, int cus);
int w8a8_choose_plan(int64_t m, int64_t n, int64_t k, int cus, int64_t ws_bytes, int* splits);
int64_t w8a8_plan_workspace(int config, int splits, int64_t m, int64_t n);
bool w8a8_plan_valid(int config, int splits, int64_t m, int64_t n, int64_t k);
void w8a8_config_geometry(int config, int32_t* out5);

// W8A8 with weight scales per group of 128 input channels, w_scale [n, k / 128]
// (k % 128 == 0), on a group-scale configuration (`config`, or -1 for the model's choice).
int w8a8_choose_gs_config(int64_t m, int64_t n, int64_t k, int cus);
hipError_t launch_w8a8_gemm_g128(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                 const float* w_scale, const float* bias, void* y,
                                 i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                 int config, hipStream_t stream);

hipError_t launch_w8a16_gemm(const void* x, const int8_t* wq, const float* w_scale,
                             const float* bias, void* y, i8ql_dtype y_dtype, int64_t m,
                             int64_t n, int64_t k, hipStream_t stream);

hipError_t launch_grouped_w8a16_gemm(const void* x, int x_per_assignment, const int8_t* wq,
                                     const float* w_scale, int64_t num_experts,
                                     const int32_t* expert_ids, int64_t t, int64_t topk,
                                     void* y, i8ql_dtype y_dtype, int64_t n, int64_t k,
                                     hipStream_t stream);

// One scale per group of 128 input channels: q [n, k], scale [n, k / 128] (k % 128 == 0).
hipError_t launch_quantize_groups128(const void* a, i8ql_dtype dtype, int64_t n, int64_t k,
                                     int8_t* q, float* scale, hipStream_t stream);

// W8A16 with w_scale [n, k / 128] (one scale per channel and group of 128 input channels).
hipError_t launch_w8a16_gemm_g128(const void* x, const int8_t* wq, const float* w_scale,
                                  const float* bias, void* y, i8ql_dtype y_dtype, int64_t m,
                                  int64_t n, int64_t k, hipStream_t stream);

// Gate/up over weights stacked [num_experts, 2n, k] (gate rows, then up rows) with the
// SiLU·mul fused: h [t * topk, n] = silu(gate) * up.
hipError_t launch_grouped_w8a16_silu_gemm(const void* x, int x_per_assignment,
                                          const int8_t* wq, const float* w_scale,
                                          int64_t num_experts, const int32_t* expert_ids,
                                          int64_t t, int64_t topk, void* h, i8ql_dtype h_dtype,
                                          int64_t n, int64_t k, hipStream_t stream);

hipError_t launch_moe_route_topk(const void* logits, i8ql_dtype dtype, int64_t t,
                                 int64_t e_routed, int64_t k_routed, int64_t n_shared,
                                 int32_t* ids, float* weights, hipStream_t stream);

hipError_t launch_moe_combine(const void* d, i8ql_dtype d_dtype, const float* weights,
                              int64_t t, int64_t topk, int64_t n, void* y, i8ql_dtype y_dtype,
                              hipStream_t stream);

}  // namespace i8ql
