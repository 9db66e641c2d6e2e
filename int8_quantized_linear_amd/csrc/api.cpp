// api.cpp — the C ABI of libi8ql: argument validation (fail closed) and kernel dispatch.
//
// Every entry point checks its arguments on the host before any HIP call, in this order:
// dtype, negative or degenerate dimensions, the zero-size no-op, NULL pointers, alignment
// and limits.  Unsupported input never reaches a kernel and never selects a different
// kernel: it returns an error, as the fail-closed scheme resolution of
// "feat(quantization): support compressed-tensors W8A8 and mixed modules" (Summary, Notes
// for Reviewers) does for unsupported checkpoints.  Only I8QL_ERR_HIP follows a launch.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "i8ql.h"
#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxElems = int64_t(1) << 62;
constexpr int64_t kMaxGridX = 2147483647;
constexpr int64_t kMaxGridY = 65535;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(i8ql_dtype d) {
  switch (d) {
    case I8QL_F32: return 4;
    case I8QL_BF16: return 2;
    case I8QL_F16: return 2;
    case I8QL_I8: return 1;
    case I8QL_I32: return 4;
  }
  return 0;
}

bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= kMaxElems / a; }

// W8A8 sizes: products within range, and one workgroup per 64 x 32 output tile (the
// smallest tile) times the most splits within a one-dimensional grid.
bool w8a8_sizes_ok(int64_t m, int64_t n, int64_t k) {
  if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n)) return false;
  const int64_t tm = (m + 63) / 64, tn = (n + 31) / 32;
  return mul_ok(tm, tn) && tm * tn <= kMaxGridX - 8;
}

i8ql_status hip_status(hipError_t e) {
  if (e == hipSuccess) return I8QL_OK;
  g_last_hip_error = static_cast<int>(e);
  return I8QL_ERR_HIP;
}

i8ql_status quantize_rows(const void* a, i8ql_dtype dtype, int64_t rows, int64_t k,
                          int8_t* q, float* scale, void* stream) {
  if (dtype != I8QL_F32 && dtype != I8QL_BF16 && dtype != I8QL_F16) return I8QL_ERR_DTYPE;
  if (rows < 0 || k < 1) return I8QL_ERR_SHAPE;
  if (!mul_ok(rows, k) || (rows + 3) / 4 > kMaxGridX) return I8QL_ERR_SHAPE;
  if (rows == 0) return I8QL_OK;
  if (!a || !q || !scale) return I8QL_ERR_NULL;
  if (!aligned(a, elem_bytes(dtype)) || !aligned(scale, 4)) return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_quantize_rows(a, dtype, rows, k, q, scale,
                                               static_cast<hipStream_t>(stream)));
}

// The RMS norm entry points: quantized (q and scale) or bf16 (h) output.
i8ql_status rmsnorm(const void* x, void* residual, const void* gamma, float eps, int64_t m,
                    int64_t k, int8_t* q, float* scale, void* h, void* stream) {
  if (m < 0 || k < 1 || k % 8 != 0 || k > I8QL_NORM_MAX_K) return I8QL_ERR_SHAPE;
  if (!mul_ok(m, k) || m > kMaxGridX) return I8QL_ERR_SHAPE;
  if (!(eps > 0.0f) || !(eps <= 3.4028234663852886e38f)) return I8QL_ERR_ARG;
  if (m == 0) return I8QL_OK;
  if (!x || !gamma || (h ? false : (!q || !scale))) return I8QL_ERR_NULL;
  if (!aligned(x, 16) || !aligned(gamma, 16) || (residual && !aligned(residual, 16)) ||
      (h && !aligned(h, 16)) || (q && !aligned(q, 8)) || (scale && !aligned(scale, 4)))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_rmsnorm(x, residual, gamma, eps, m, k, q, scale, h,
                                         static_cast<hipStream_t>(stream)));
}

// The SiLU·mul entry points: quantized (q and scale) or bf16 (h) output.
i8ql_status silu_mul(const void* gu, int64_t m, int64_t n, int8_t* q, float* scale, void* h,
                     void* stream) {
  if (m < 0 || n < 1 || n % 8 != 0 || n > I8QL_SILU_MAX_N) return I8QL_ERR_SHAPE;
  if (!mul_ok(m, 2 * n) || m > kMaxGridX) return I8QL_ERR_SHAPE;
  if (m == 0) return I8QL_OK;
  if (!gu || (h ? false : (!q || !scale))) return I8QL_ERR_NULL;
  if (!aligned(gu, 16) || (h && !aligned(h, 16)) || (q && !aligned(q, 8)) ||
      (scale && !aligned(scale, 4)))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_silu_mul(gu, m, n, q, scale, h,
                                          static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

i8ql_status quantize_per_channel_int8(const void* w, i8ql_dtype w_dtype, int64_t n, int64_t k,
                                      int8_t* q_out, float* scale_out, void* stream) {
  return quantize_rows(w, w_dtype, n, k, q_out, scale_out, stream);
}

i8ql_status quantize_per_token_int8(const void* x, i8ql_dtype x_dtype, int64_t m, int64_t k,
                                    int8_t* q_out, float* scale_out, void* stream) {
  return quantize_rows(x, x_dtype, m, k, q_out, scale_out, stream);
}

i8ql_status quantize_per_token_int8_multi(const i8ql_quant_job* jobs, int count,
                                          i8ql_dtype x_dtype, void* stream) {
  if (!jobs || count < 1 || count > I8QL_QUANT_MAX_JOBS) return I8QL_ERR_ARG;
  if (x_dtype != I8QL_F32 && x_dtype != I8QL_BF16 && x_dtype != I8QL_F16) return I8QL_ERR_DTYPE;
  const int eb = elem_bytes(x_dtype);
  for (int i = 0; i < count; ++i) {
    const i8ql_quant_job& j = jobs[i];
    if (j.rows < 0 || j.k < 1 || !mul_ok(j.rows, j.k) || j.rows > kMaxGridX)
      return I8QL_ERR_SHAPE;
  }
  for (int i = 0; i < count; ++i) {
    const i8ql_quant_job& j = jobs[i];
    if (j.rows == 0) continue;
    if (!j.x || !j.q_out || !j.scale_out) return I8QL_ERR_NULL;
    if (!aligned(j.x, 16) || (j.k * eb) % 16 != 0 || !aligned(j.q_out, 8) ||
        !aligned(j.scale_out, 4))
      return I8QL_ERR_ALIGN;
  }
  return hip_status(i8ql::launch_quantize_rows_multi(jobs, count, x_dtype,
                                                     static_cast<hipStream_t>(stream)));
}

i8ql_status rmsnorm_quantize_per_token_int8(const void* x, void* residual, const void* gamma,
                                            float eps, int64_t m, int64_t k, int8_t* q_out,
                                            float* scale_out, void* stream) {
  return rmsnorm(x, residual, gamma, eps, m, k, q_out, scale_out, nullptr, stream);
}

i8ql_status rmsnorm_bf16(const void* x, void* residual, const void* gamma, float eps, int64_t m,
                         int64_t k, void* y_out, void* stream) {
  return rmsnorm(x, residual, gamma, eps, m, k, nullptr, nullptr, y_out, stream);
}

i8ql_status silu_mul_quantize_per_token_int8(const void* gu, int64_t m, int64_t n,
                                             int8_t* q_out, float* scale_out, void* stream) {
  return silu_mul(gu, m, n, q_out, scale_out, nullptr, stream);
}

i8ql_status silu_mul_bf16(const void* gu, int64_t m, int64_t n, void* h_out, void* stream) {
  return silu_mul(gu, m, n, nullptr, nullptr, h_out, stream);
}

}  // extern "C"

namespace {

// Validation shared by the plan entry points; `workspace_bytes` is the workspace the plan may
// use (the caller's, or the static scratch).  Returns I8QL_OK when the call may launch, or
// the status to return (also I8QL_OK with *noop set for an empty product).
i8ql_status w8a8_validate(int config, int splits, const int8_t* xq, const float* x_scale,
                          const int8_t* wq, const float* w_scale, const float* bias,
                          const void* y, i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                          bool has_workspace, int64_t workspace_bytes, bool* noop) {
  *noop = false;
  if (y_dtype != I8QL_BF16 && y_dtype != I8QL_F32 && y_dtype != I8QL_I32) return I8QL_ERR_DTYPE;
  if (m < 0 || n < 0 || k < 1) return I8QL_ERR_SHAPE;
  if (!w8a8_sizes_ok(m, n, k)) return I8QL_ERR_SHAPE;
  if (config < -1 || config >= I8QL_W8A8_NUM_CONFIGS || workspace_bytes < 0) return I8QL_ERR_ARG;
  if (config == -1 ? splits != -1 : (splits < 1 || splits > I8QL_W8A8_MAX_SPLITS))
    return I8QL_ERR_ARG;
  if (config >= 0) {
    int32_t geo[5];
    i8ql::w8a8_config_geometry(config, geo);
    if (k % (128 * static_cast<int64_t>(geo[2])) != 0 && geo[2] > 1) return I8QL_ERR_ARG;
    if (splits > 1 && (!geo[3] || splits > (k + 127) / 128)) return I8QL_ERR_ARG;
    if (splits > 1 && !i8ql::w8a8_plan_valid(config, splits, m, n, k)) return I8QL_ERR_SHAPE;
  }
  if (m == 0 || n == 0) {
    *noop = true;
    return I8QL_OK;
  }
  if (!xq || !wq || !y) return I8QL_ERR_NULL;
  if (y_dtype != I8QL_I32 && (!x_scale || !w_scale)) return I8QL_ERR_NULL;
  if (y_dtype == I8QL_I32 && bias) return I8QL_ERR_ARG;
  if (k % 16 != 0 || !aligned(xq, 16) || !aligned(wq, 16)) return I8QL_ERR_ALIGN;
  if (!aligned(y, elem_bytes(y_dtype)) || !aligned(x_scale, 4) || !aligned(w_scale, 4) ||
      !aligned(bias, 4))
    return I8QL_ERR_ALIGN;
  if (k > I8QL_W8A8_MAX_K) return I8QL_ERR_K_TOO_LARGE;
  if (config >= 0) {
    const int64_t need = i8ql::w8a8_plan_workspace(config, splits, m, n);
    if (need > 0 && !has_workspace) return I8QL_ERR_NULL;
    if (need > workspace_bytes) return I8QL_ERR_WORKSPACE;
  }
  return I8QL_OK;
}

}  // namespace

extern "C" {

i8ql_status w8a8_gemm_with_plan(int config, int splits, const int8_t* xq, const float* x_scale,
                                const int8_t* wq, const float* w_scale, const float* bias,
                                void* y, i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                void* workspace, int64_t workspace_bytes, void* stream) {
  if (workspace_bytes < 0) return I8QL_ERR_ARG;
  if (!workspace) workspace_bytes = 0;
  bool noop = false;
  const i8ql_status st = w8a8_validate(config, splits, xq, x_scale, wq, w_scale, bias, y,
                                       y_dtype, m, n, k, workspace != nullptr, workspace_bytes,
                                       &noop);
  if (st != I8QL_OK || noop) return st;
  if (workspace && !aligned(workspace, 16)) return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_w8a8_gemm(xq, x_scale, wq, w_scale, bias, y, y_dtype, m, n, k,
                                           config, splits, workspace, workspace_bytes,
                                           static_cast<hipStream_t>(stream)));
}

i8ql_status w8a8_gemm_noalloc(int config, int splits, const int8_t* xq, const float* x_scale,
                              const int8_t* wq, const float* w_scale, const float* bias, void* y,
                              i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                              void* stream) {
  bool noop = false;
  const i8ql_status st = w8a8_validate(config, splits, xq, x_scale, wq, w_scale, bias, y,
                                       y_dtype, m, n, k, true, I8QL_W8A8_SCRATCH_BYTES, &noop);
  if (st != I8QL_OK || noop) return st;
  return hip_status(i8ql::launch_w8a8_gemm_noalloc(xq, x_scale, wq, w_scale, bias, y, y_dtype,
                                                   m, n, k, config, splits,
                                                   static_cast<hipStream_t>(stream)));
}

i8ql_status w8a8_gemm_with_config(int config, const int8_t* xq, const float* x_scale,
                                  const int8_t* wq, const float* w_scale, const float* bias,
                                  void* y, i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                  void* stream) {
  return w8a8_gemm_with_plan(config, config < 0 ? -1 : 1, xq, x_scale, wq, w_scale, bias, y,
                             y_dtype, m, n, k, nullptr, 0, stream);
}

i8ql_status w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                      const float* w_scale, const float* bias, void* y, i8ql_dtype y_dtype,
                      int64_t m, int64_t n, int64_t k, void* stream) {
  return w8a8_gemm_with_plan(-1, -1, xq, x_scale, wq, w_scale, bias, y, y_dtype, m, n, k,
                             nullptr, 0, stream);
}

i8ql_status w8a8_gemm_config_info(int config, int32_t* out5) {
  if (!out5) return I8QL_ERR_NULL;
  if (config < 0 || config >= I8QL_W8A8_NUM_CONFIGS) return I8QL_ERR_ARG;
  i8ql::w8a8_config_geometry(config, out5);
  return I8QL_OK;
}

i8ql_status w8a8_gemm_g128_with_config(int config, const int8_t* xq, const float* x_scale,
                                       const int8_t* wq, const float* w_scale,
                                       const float* bias, void* y, i8ql_dtype y_dtype,
                                       int64_t m, int64_t n, int64_t k, void* stream) {
  if (y_dtype != I8QL_BF16 && y_dtype != I8QL_F32) return I8QL_ERR_DTYPE;
  if (m < 0 || n < 0 || k < 1 || k % I8QL_GROUP_SIZE != 0) return I8QL_ERR_SHAPE;
  if (!w8a8_sizes_ok(m, n, k)) return I8QL_ERR_SHAPE;
  if (config < -1 || config >= I8QL_W8A8_NUM_CONFIGS) return I8QL_ERR_ARG;
  if (config >= 0) {
    int32_t geo[5];
    i8ql::w8a8_config_geometry(config, geo);
    if (!geo[4]) return I8QL_ERR_ARG;
  }
  if (m == 0 || n == 0) return I8QL_OK;
  if (!xq || !wq || !y || !x_scale || !w_scale) return I8QL_ERR_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16)) return I8QL_ERR_ALIGN;
  if (!aligned(y, elem_bytes(y_dtype)) || !aligned(x_scale, 4) || !aligned(w_scale, 4) ||
      !aligned(bias, 4))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_w8a8_gemm_g128(xq, x_scale, wq, w_scale, bias, y, y_dtype, m, n,
                                                k, config, static_cast<hipStream_t>(stream)));
}

i8ql_status w8a8_gemm_g128(const int8_t* xq, const float* x_scale, const int8_t* wq,
                           const float* w_scale, const float* bias, void* y, i8ql_dtype y_dtype,
                           int64_t m, int64_t n, int64_t k, void* stream) {
  return w8a8_gemm_g128_with_config(-1, xq, x_scale, wq, w_scale, bias, y, y_dtype, m, n, k,
                                    stream);
}

int w8a8_gemm_choose_config(int64_t m, int64_t n, int64_t k, int cus) {
  if (m < 1 || n < 1 || k < 16 || k % 16 != 0 || k > I8QL_W8A8_MAX_K || cus < 1) return -1;
  if (!w8a8_sizes_ok(m, n, k)) return -1;
  return i8ql::w8a8_choose_config(m, n, k, cus);
}

i8ql_status w8a8_gemm_choose_plan(int64_t m, int64_t n, int64_t k, int cus,
                                  int64_t workspace_bytes, int32_t* out2) {
  if (!out2) return I8QL_ERR_NULL;
  if (m < 1 || n < 1 || k < 16 || k % 16 != 0 || k > I8QL_W8A8_MAX_K || cus < 1 ||
      workspace_bytes < 0 || !w8a8_sizes_ok(m, n, k))
    return I8QL_ERR_ARG;
  int sp = 1;
  out2[0] = i8ql::w8a8_choose_plan(m, n, k, cus, workspace_bytes, &sp);
  out2[1] = sp;
  return I8QL_OK;
}

int64_t w8a8_gemm_workspace_size(int config, int splits, int64_t m, int64_t n, int64_t k,
                                 int cus) {
  if (m < 1 || n < 1 || k < 16 || k % 16 != 0 || k > I8QL_W8A8_MAX_K || cus < 1 ||
      !w8a8_sizes_ok(m, n, k))
    return -1;
  if (config == -1 && splits == -1) {
    int sp = 1;
    const int c = i8ql::w8a8_choose_plan(m, n, k, cus, INT64_MAX, &sp);
    return i8ql::w8a8_plan_workspace(c, sp, m, n);
  }
  if (config < 0 || config >= I8QL_W8A8_NUM_CONFIGS || splits < 1 ||
      splits > I8QL_W8A8_MAX_SPLITS || !i8ql::w8a8_plan_valid(config, splits, m, n, k))
    return -1;
  return i8ql::w8a8_plan_workspace(config, splits, m, n);
}

i8ql_status w8a16_gemm(const void* x, const int8_t* wq, const float* w_scale, const float* bias,
                       void* y, i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                       void* stream) {
  if (y_dtype != I8QL_BF16 && y_dtype != I8QL_F32) return I8QL_ERR_DTYPE;
  if (m < 0 || n < 0 || k < 1) return I8QL_ERR_SHAPE;
  if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n)) return I8QL_ERR_SHAPE;
  if ((n + 15) / 16 > kMaxGridX || (m + 63) / 64 > kMaxGridY) return I8QL_ERR_SHAPE;
  if (m == 0 || n == 0) return I8QL_OK;
  if (!x || !wq || !w_scale || !y) return I8QL_ERR_NULL;
  if (k % 16 != 0 || !aligned(x, 16) || !aligned(wq, 16)) return I8QL_ERR_ALIGN;
  if (!aligned(y, elem_bytes(y_dtype)) || !aligned(w_scale, 4) || !aligned(bias, 4))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_w8a16_gemm(x, wq, w_scale, bias, y, y_dtype, m, n, k,
                                            static_cast<hipStream_t>(stream)));
}

i8ql_status grouped_w8a16_gemm(const void* x, int x_per_assignment, const int8_t* wq,
                               const float* w_scale, int64_t num_experts,
                               const int32_t* expert_ids, int64_t t, int64_t topk, void* y,
                               i8ql_dtype y_dtype, int64_t n, int64_t k, void* stream) {
  if (y_dtype != I8QL_BF16 && y_dtype != I8QL_F32) return I8QL_ERR_DTYPE;
  if (x_per_assignment != 0 && x_per_assignment != 1) return I8QL_ERR_ARG;
  if (topk < 1 || topk > 64 || num_experts < 1 || num_experts > kMaxGridY - 1) return I8QL_ERR_ARG;
  if (t < 0 || n < 0 || k < 1) return I8QL_ERR_SHAPE;
  if (t * topk > 65536 || k > I8QL_GROUPED_MAX_K) return I8QL_ERR_SHAPE;
  if (!mul_ok(num_experts, n) || !mul_ok(num_experts * n, k) || !mul_ok(t * topk, k) ||
      !mul_ok(t * topk, n) || (n + 15) / 16 > kMaxGridX)
    return I8QL_ERR_SHAPE;
  if (t == 0 || n == 0) return I8QL_OK;
  if (!x || !wq || !w_scale || !expert_ids || !y) return I8QL_ERR_NULL;
  if (k % 16 != 0 || !aligned(x, 16) || !aligned(wq, 16)) return I8QL_ERR_ALIGN;
  if (!aligned(y, elem_bytes(y_dtype)) || !aligned(w_scale, 4) || !aligned(expert_ids, 4))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_grouped_w8a16_gemm(x, x_per_assignment, wq, w_scale,
                                                    num_experts, expert_ids, t, topk, y,
                                                    y_dtype, n, k,
                                                    static_cast<hipStream_t>(stream)));
}

i8ql_status quantize_per_group_int8(const void* w, i8ql_dtype w_dtype, int64_t n, int64_t k,
                                    int8_t* q_out, float* scale_out, void* stream) {
  if (w_dtype != I8QL_F32 && w_dtype != I8QL_BF16 && w_dtype != I8QL_F16) return I8QL_ERR_DTYPE;
  if (n < 0 || k < 1 || k % I8QL_GROUP_SIZE != 0) return I8QL_ERR_SHAPE;
  if (!mul_ok(n, k) || n * k / 8 / 256 >= kMaxGridX) return I8QL_ERR_SHAPE;
  if (n == 0) return I8QL_OK;
  if (!w || !q_out || !scale_out) return I8QL_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q_out, 8) || !aligned(scale_out, 4)) return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_quantize_groups128(w, w_dtype, n, k, q_out, scale_out,
                                                    static_cast<hipStream_t>(stream)));
}

i8ql_status w8a16_gemm_g128(const void* x, const int8_t* wq, const float* w_scale,
                            const float* bias, void* y, i8ql_dtype y_dtype, int64_t m,
                            int64_t n, int64_t k, void* stream) {
  if (y_dtype != I8QL_BF16 && y_dtype != I8QL_F32) return I8QL_ERR_DTYPE;
  if (m < 0 || n < 0 || k < 1 || k % I8QL_GROUP_SIZE != 0) return I8QL_ERR_SHAPE;
  if (!mul_ok(m, k) || !mul_ok(n, k) || !mul_ok(m, n)) return I8QL_ERR_SHAPE;
  if ((n + 15) / 16 > kMaxGridX || (m + 63) / 64 > kMaxGridY) return I8QL_ERR_SHAPE;
  if (m == 0 || n == 0) return I8QL_OK;
  if (!x || !wq || !w_scale || !y) return I8QL_ERR_NULL;
  if (!aligned(x, 16) || !aligned(wq, 16)) return I8QL_ERR_ALIGN;
  if (!aligned(y, elem_bytes(y_dtype)) || !aligned(w_scale, 4) || !aligned(bias, 4))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_w8a16_gemm_g128(x, wq, w_scale, bias, y, y_dtype, m, n, k,
                                                 static_cast<hipStream_t>(stream)));
}

i8ql_status grouped_w8a16_silu_gemm(const void* x, int x_per_assignment, const int8_t* wq,
                                    const float* w_scale, int64_t num_experts,
                                    const int32_t* expert_ids, int64_t t, int64_t topk, void* h,
                                    i8ql_dtype h_dtype, int64_t n, int64_t k, void* stream) {
  if (h_dtype != I8QL_BF16 && h_dtype != I8QL_F32) return I8QL_ERR_DTYPE;
  if (x_per_assignment != 0 && x_per_assignment != 1) return I8QL_ERR_ARG;
  if (topk < 1 || topk > 64 || num_experts < 1 || num_experts > kMaxGridY - 1) return I8QL_ERR_ARG;
  if (t < 0 || n < 0 || k < 1) return I8QL_ERR_SHAPE;
  if (t * topk > 65536 || k > I8QL_GROUPED_MAX_K) return I8QL_ERR_SHAPE;
  if (!mul_ok(num_experts, 2 * n) || !mul_ok(num_experts * 2 * n, k) || !mul_ok(t * topk, k) ||
      !mul_ok(t * topk, n) || (n + 15) / 16 > kMaxGridX)
    return I8QL_ERR_SHAPE;
  if (t == 0 || n == 0) return I8QL_OK;
  if (!x || !wq || !w_scale || !expert_ids || !h) return I8QL_ERR_NULL;
  if (k % 16 != 0 || !aligned(x, 16) || !aligned(wq, 16)) return I8QL_ERR_ALIGN;
  if (!aligned(h, elem_bytes(h_dtype)) || !aligned(w_scale, 4) || !aligned(expert_ids, 4))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_grouped_w8a16_silu_gemm(
      x, x_per_assignment, wq, w_scale, num_experts, expert_ids, t, topk, h, h_dtype, n, k,
      static_cast<hipStream_t>(stream)));
}

i8ql_status moe_route_topk(const void* logits, i8ql_dtype logits_dtype, int64_t t,
                           int64_t e_routed, int64_t k_routed, int64_t n_shared, int32_t* ids,
                           float* weights, void* stream) {
  if (logits_dtype != I8QL_F32 && logits_dtype != I8QL_BF16) return I8QL_ERR_DTYPE;
  if (t < 0 || t > kMaxGridX) return I8QL_ERR_SHAPE;
  if (e_routed < 1 || e_routed > I8QL_ROUTE_MAX_EXPERTS || k_routed < 1 ||
      k_routed > I8QL_ROUTE_MAX_K || k_routed > e_routed || n_shared < 0 ||
      n_shared > I8QL_ROUTE_MAX_K || k_routed + n_shared > 64)
    return I8QL_ERR_ARG;
  if (!mul_ok(t, e_routed) || !mul_ok(t, k_routed + n_shared)) return I8QL_ERR_SHAPE;
  if (t == 0) return I8QL_OK;
  if (!logits || !ids || !weights) return I8QL_ERR_NULL;
  if (!aligned(logits, elem_bytes(logits_dtype)) || !aligned(ids, 4) || !aligned(weights, 4))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_moe_route_topk(logits, logits_dtype, t, e_routed, k_routed,
                                                n_shared, ids, weights,
                                                static_cast<hipStream_t>(stream)));
}

i8ql_status moe_combine(const void* d, i8ql_dtype d_dtype, const float* weights, int64_t t,
                        int64_t topk, int64_t n, void* y, i8ql_dtype y_dtype, void* stream) {
  if ((d_dtype != I8QL_BF16 && d_dtype != I8QL_F32) ||
      (y_dtype != I8QL_BF16 && y_dtype != I8QL_F32))
    return I8QL_ERR_DTYPE;
  if (topk < 1 || topk > 64) return I8QL_ERR_ARG;
  if (t < 0 || n < 0 || t > kMaxGridX || (n + 255) / 256 > kMaxGridY) return I8QL_ERR_SHAPE;
  if (!mul_ok(t * topk, n)) return I8QL_ERR_SHAPE;
  if (t == 0 || n == 0) return I8QL_OK;
  if (!d || !weights || !y) return I8QL_ERR_NULL;
  if (!aligned(d, elem_bytes(d_dtype)) || !aligned(y, elem_bytes(y_dtype)) ||
      !aligned(weights, 4))
    return I8QL_ERR_ALIGN;
  return hip_status(i8ql::launch_moe_combine(d, d_dtype, weights, t, topk, n, y, y_dtype,
                                             static_cast<hipStream_t>(stream)));
}

const char* i8ql_status_string(i8ql_status s) {
  switch (s) {
    case I8QL_OK: return "I8QL_OK";
    case I8QL_ERR_NULL: return "I8QL_ERR_NULL";
    case I8QL_ERR_SHAPE: return "I8QL_ERR_SHAPE";
    case I8QL_ERR_DTYPE: return "I8QL_ERR_DTYPE";
    case I8QL_ERR_ALIGN: return "I8QL_ERR_ALIGN";
    case I8QL_ERR_K_TOO_LARGE: return "I8QL_ERR_K_TOO_LARGE";
    case I8QL_ERR_ARG: return "I8QL_ERR_ARG";
    case I8QL_ERR_HIP: return "I8QL_ERR_HIP";
    case I8QL_ERR_WORKSPACE: return "I8QL_ERR_WORKSPACE";
  }
  return "I8QL_UNKNOWN_STATUS";
}

int i8ql_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
