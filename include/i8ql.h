/*
 * i8ql.h — C ABI of the int8 quantized linear layer for AMD Instinct MI355X (gfx950).
 *
 * The operations follow three web pages:
 *   [P5a]   "Phase 5a: int8 weight-only quantization" (dispatch pull request #5), Summary.
 *   [W8A8]  "feat(quantization): support compressed-tensors W8A8 and mixed modules"
 *           (InfiniLM pull request #582), section "Design and Supported Execution Scheme".
 *   [Day6]  "Day 6 — Quantize It Yourself", section "The mechanism", blocks 1 and 5.
 *
 * Conventions shared by every entry point
 *   - Pointers named as device pointers must point to device memory (or memory the device
 *     can access); host-side arguments are plain integers and enums.
 *   - Every tensor is dense and row-major with no padding: a [R, C] tensor has row stride C
 *     elements.  Weights use the nn.Linear layout [N, K] (output channel, input channel);
 *     activations are [M, K] (one row per token).  Y = X * W^T has shape [M, N].
 *   - Ownership: the caller owns every buffer, including the W8A8 workspace.  The library
 *     allocates no device or host memory, keeps no pointer after a call returns and holds
 *     no mutable global state apart from the thread-local error slot read by
 *     i8ql_last_hip_error() and per-device caches of launch settings (set once, idempotent).
 *   - Asynchrony: a call validates its arguments on the host, enqueues its kernels on
 *     `stream` (a hipStream_t passed as void*; NULL selects the null stream) and returns.
 *     It never synchronizes.  Results are ready once the stream reaches that point.
 *   - Errors fail closed: an unsupported dtype, shape, alignment or combination returns an
 *     error code before any device work, and the outputs are left untouched.  There is no
 *     fallback path.  Only I8QL_ERR_HIP can follow a launch attempt.
 *   - A zero dimension (m, n, t or the row count) makes the call a no-op returning I8QL_OK.
 *     Negative dimensions return I8QL_ERR_SHAPE.
 *   - Outputs must not overlap inputs or each other.
 *   - Results are deterministic: the same inputs give bitwise the same outputs on every
 *     call (the only atomics count arrivals; no output value depends on their order).
 *   - Inputs must be finite; NaN or Inf inputs give unspecified (but in-bounds) results.
 */
#ifndef I8QL_H
#define I8QL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  I8QL_F32 = 0,  /* IEEE binary32 */
  I8QL_BF16 = 1, /* bfloat16 (upper half of binary32) */
  I8QL_F16 = 2,  /* IEEE binary16 */
  I8QL_I8 = 3,   /* signed 8-bit integer */
  I8QL_I32 = 4   /* signed 32-bit integer */
} i8ql_dtype;

typedef enum {
  I8QL_OK = 0,
  I8QL_ERR_NULL = 1,        /* a required pointer is NULL */
  I8QL_ERR_SHAPE = 2,       /* a dimension is negative, or k < 1, or a size overflows */
  I8QL_ERR_DTYPE = 3,       /* a dtype this entry point does not accept */
  I8QL_ERR_ALIGN = 4,       /* GEMM: k % 16 != 0, or an operand base pointer is not 16-byte aligned */
  I8QL_ERR_K_TOO_LARGE = 5, /* w8a8_gemm: k > 133144, so an int32 accumulator could overflow */
  I8QL_ERR_ARG = 6,         /* invalid combination: bias with I32 output, topk < 1, experts < 1, ... */
  I8QL_ERR_HIP = 7,         /* the HIP runtime reported an error; see i8ql_last_hip_error() */
  I8QL_ERR_WORKSPACE = 8    /* the requested W8A8 plan needs more workspace than was given */
} i8ql_status;

/* Largest K for which k * 127 * 127 fits in a signed 32-bit accumulator (133144 * 16129 =
 * 2147479576 < 2^31). */
#define I8QL_W8A8_MAX_K 133144

/*
 * quantize_per_channel_int8 — symmetric per-output-channel int8 weight quantization.
 *
 * Defines: [Day6] block 1 (codes q = clamp(round(w / s)), shared scale s = absmax of the
 * group / largest representable code, reconstruction w ~ s * q, one scale per output
 * channel); [P5a] Summary (the quantizer of the grouped int8 kernel; its second bug fix puts
 * the arithmetic in float32, its third limits the zero-channel guard to all-zero channels);
 * [W8A8] "Design and Supported Execution Scheme" (static symmetric INT8 per-channel weights).
 *
 * For each row r of w[n, k] (one output channel):
 *   amax = max_j |w[r, j]|  (inputs widened exactly to float32)
 *   s    = amax / 127        (float32 division, round to nearest even)
 *   if s == 0:  scale_out[r] = 1.0f and q_out[r, :] = 0      (all-zero channel guard)
 *   else:       q_out[r, j] = clamp(rne(w[r, j] / s), -127, 127) (float32 division per
 *               element, ties to even); scale_out[r] = s.
 *   The code -128 is never produced.
 *
 * w          device, [n, k] of w_dtype in {I8QL_F32, I8QL_BF16, I8QL_F16}, element-aligned.
 * q_out      device, [n, k] int8.       scale_out  device, [n] float32.
 * n >= 0 rows, k >= 1 columns; n * k < 2^62.
 * Errors: NULL pointer -> I8QL_ERR_NULL; n < 0 or k < 1 -> I8QL_ERR_SHAPE; other dtype ->
 * I8QL_ERR_DTYPE; a pointer not aligned to its element size -> I8QL_ERR_ALIGN.
 */
i8ql_status quantize_per_channel_int8(const void* w, i8ql_dtype w_dtype, int64_t n, int64_t k,
                                      int8_t* q_out, float* scale_out, void* stream);

/*
 * quantize_per_token_int8 — dynamic symmetric per-token int8 activation quantization.
 *
 * Defines: [W8A8] "Design and Supported Execution Scheme" (dynamic symmetric INT8 per-token
 * input activations); [Day6] block 5 (activations quantized on the fly with per-token
 * dynamic scales) and "Reading-share post" fact 2 (each token's scale is computed at run
 * time, an extra step of every forward pass).
 *
 * Exactly the row rule of quantize_per_channel_int8, applied to each row (token) of x[m, k]:
 * one float32 scale per token.  Arguments as above with m rows.
 */
i8ql_status quantize_per_token_int8(const void* x, i8ql_dtype x_dtype, int64_t m, int64_t k,
                                    int8_t* q_out, float* scale_out, void* stream);

/*
 * quantize_per_token_int8_multi — quantize_per_token_int8 of up to I8QL_QUANT_MAX_JOBS
 * independent activation matrices of one dtype in a single launch (one kernel instead of one
 * per matrix; each matrix's codes and scales are bitwise those quantize_per_token_int8
 * writes).  For callers that hold several activation tensors at once; the per-token scale
 * is computed at run time for each of them ([W8A8] "Design and Supported Execution Scheme";
 * [Day6] "Reading-share post" fact 2: the extra work of every forward pass).
 *
 * jobs   host, `count` descriptors: x (device, [rows, k] of x_dtype), rows >= 0, k >= 1,
 *        q_out (device, [rows, k] int8), scale_out (device, [rows] float32).  The matrices
 *        must not overlap one another's outputs.
 * 1 <= count <= I8QL_QUANT_MAX_JOBS; x_dtype in {I8QL_F32, I8QL_BF16, I8QL_F16}.
 * Every x is 16-byte aligned with k * element size a multiple of 16, q_out 8-byte aligned
 * (the vector layout; quantize_per_token_int8 takes any other layout).
 * Errors: count or NULL jobs -> I8QL_ERR_ARG; dtype -> I8QL_ERR_DTYPE; a job's rows < 0, k < 1
 * or sizes out of range -> I8QL_ERR_SHAPE; a NULL pointer of a non-empty job -> I8QL_ERR_NULL;
 * alignment -> I8QL_ERR_ALIGN.  Nothing is launched unless every job is valid.
 */
#define I8QL_QUANT_MAX_JOBS 8
typedef struct {
  const void* x;
  int64_t rows;
  int64_t k;
  int8_t* q_out;
  float* scale_out;
} i8ql_quant_job;
i8ql_status quantize_per_token_int8_multi(const i8ql_quant_job* jobs, int count,
                                          i8ql_dtype x_dtype, void* stream);

/*
 * rmsnorm_quantize_per_token_int8 — the per-token int8 quantization of a projection's input
 * fused into the RMS norm that produces it, so the activations make one trip through HBM
 * as int8 codes instead of a bf16 write and read before the quantizer.
 *
 * Defines: [W8A8] "Design and Supported Execution Scheme" (dynamic symmetric INT8 per-token
 * input activations) and its "Weight footprint" section (normalization weights stay in
 * higher precision); [Day6] "Reading-share post" fact 2 (the per-token scale is extra work
 * of every forward pass).  The norm is not written out on the pages; the reading used, per
 * row i of k elements (bf16 inputs widened exactly to float32):
 *   u = x[i, :], or with a residual stream u = bf16(x[i, :] + residual[i, :]) (one float32
 *       addition rounded to nearest even), which is also written back to residual[i, :];
 *   S = sum_j u_j^2 in float64;  v = fl32(S / k);
 *   r = fl32(1 / fl32(sqrt(fl32(v + eps))))  (correctly rounded float32 operations);
 *   h_j = bf16(fl32(fl32(u_j * r) * gamma[j]));
 * then the row rule of quantize_per_channel_int8 on h: scale_out[i], q_out[i, :].  The
 * codes and scales are bitwise those of rmsnorm_bf16 followed by quantize_per_token_int8.
 * (The float64 sum makes the mean independent of the summation order except within about
 * 2^-50 of a float32 rounding midpoint.)
 *
 * x          device, [m, k] bf16, 16-byte aligned.
 * residual   device, [m, k] bf16, 16-byte aligned, read and overwritten with u; or NULL.
 *            Must not overlap x or the outputs.
 * gamma      device, [k] bf16 norm weights, 16-byte aligned.
 * eps        > 0 and finite.
 * q_out      device, [m, k] int8, 8-byte aligned.   scale_out  device, [m] float32.
 * m >= 0; 8 <= k <= I8QL_NORM_MAX_K with k % 8 == 0.
 * Errors: NULL x, gamma, q_out or scale_out -> I8QL_ERR_NULL; m < 0, k < 1, k % 8 != 0 or
 * k > I8QL_NORM_MAX_K -> I8QL_ERR_SHAPE; eps not finite or <= 0 -> I8QL_ERR_ARG; alignment ->
 * I8QL_ERR_ALIGN.
 */
#define I8QL_NORM_MAX_K 24576
i8ql_status rmsnorm_quantize_per_token_int8(const void* x, void* residual, const void* gamma,
                                            float eps, int64_t m, int64_t k, int8_t* q_out,
                                            float* scale_out, void* stream);

/*
 * rmsnorm_bf16 — the same RMS norm (and residual update) writing h as bf16 y_out [m, k]
 * (16-byte aligned, must not overlap the inputs): the unfused producer, whose output
 * quantize_per_token_int8 turns into exactly the codes and scales of
 * rmsnorm_quantize_per_token_int8.  Arguments and errors as there (y_out in place of q_out
 * and scale_out).
 */
i8ql_status rmsnorm_bf16(const void* x, void* residual, const void* gamma, float eps, int64_t m,
                         int64_t k, void* y_out, void* stream);

/*
 * silu_mul_quantize_per_token_int8 — the per-token int8 quantization of a down projection's
 * input fused into the SiLU·mul that produces it from the gate/up projection's output, so
 * the activation reaches HBM once, as int8 codes, instead of as bf16 written and read back.
 *
 * Defines: [W8A8] "Design and Supported Execution Scheme" (dynamic symmetric INT8 per-token
 * input activations); [Day6] "Reading-share post" fact 2 (the per-token scale is extra work
 * of every forward pass).  The activation is the one of the mixture-of-experts block's
 * grouped_w8a16_silu_gemm (not written out on the pages; reading): per row i and column j,
 *   h[i, j] = bf16(g * rcp(1 + e^-g) * u),  g = gu[i, j], u = gu[i, n + j] (bf16 widened),
 * in float32 (the hardware exponential for g >= -16; float64 where g < -80 or the nonzero
 * product is below 2^-120 in magnitude), rounded to nearest even; then the row rule of
 * quantize_per_channel_int8 on h.
 * The codes and scales are bitwise those of silu_mul_bf16 followed by
 * quantize_per_token_int8.  (h lies within about 2^-19 (relative) of the exact value, so its
 * bf16 rounding is that of the exact value except within that distance of a halfway point.)
 *
 * gu         device, [m, 2n] bf16, 16-byte aligned: the gate values in columns [0, n), the
 *            up values in [n, 2n) (the output of one GEMM over gate and up weights stacked).
 * q_out      device, [m, n] int8, 8-byte aligned.   scale_out  device, [m] float32.
 * m >= 0; 8 <= n <= I8QL_SILU_MAX_N with n % 8 == 0.
 * Errors: NULL gu, q_out or scale_out -> I8QL_ERR_NULL; m < 0, n < 1, n % 8 != 0 or
 * n > I8QL_SILU_MAX_N -> I8QL_ERR_SHAPE; alignment -> I8QL_ERR_ALIGN.
 */
#define I8QL_SILU_MAX_N 24576
i8ql_status silu_mul_quantize_per_token_int8(const void* gu, int64_t m, int64_t n,
                                             int8_t* q_out, float* scale_out, void* stream);

/*
 * silu_mul_bf16 — the same SiLU·mul writing h as bf16 h_out [m, n] (16-byte aligned, must not
 * overlap gu): the unfused producer, whose output quantize_per_token_int8 turns into exactly
 * the codes and scales of silu_mul_quantize_per_token_int8.  Arguments and errors as there.
 */
i8ql_status silu_mul_bf16(const void* gu, int64_t m, int64_t n, void* h_out, void* stream);

/*
 * w8a8_gemm — int8 x int8 GEMM with int32 accumulation and a fused scale epilogue.
 *
 * Defines: [W8A8] "Design and Supported Execution Scheme" (per-channel int8 weights,
 * per-token int8 activations, no quantization of the output); [Day6] block 5 (W8A8: both
 * operands 8-bit, the product runs on 8-bit matrix units).  Biases travel with the output
 * channels ([W8A8] Summary: scales and biases shard together by output channel).
 *
 *   acc[i, j] = sum_c xq[i, c] * wq[j, c]                  (exact, int32)
 *   y_dtype == I8QL_I32 :  y[i, j] = acc[i, j]              (bias must be NULL)
 *   otherwise           :  y[i, j] = ((float)acc * x_scale[i]) * w_scale[j] (+ bias[j]),
 *                          float32 arithmetic, then stored as float32 (I8QL_F32) or rounded
 *                          to nearest even bfloat16 (I8QL_BF16).
 *
 * xq       device, [m, k] int8, 16-byte aligned.   x_scale  device, [m] float32.
 * wq       device, [n, k] int8, 16-byte aligned.   w_scale  device, [n] float32.
 * bias     device, [n] float32, or NULL.
 * y        device, [m, n] of y_dtype in {I8QL_BF16, I8QL_F32, I8QL_I32}.
 * m, n >= 0; 16 <= k <= 133144 and k % 16 == 0.
 * Errors: NULL (x_scale/w_scale may be NULL only with I32 output) -> I8QL_ERR_NULL;
 * negative m/n, k < 1, or more than 2^31 - 9 output tiles of 64 x 32 -> I8QL_ERR_SHAPE;
 * k % 16 or misaligned xq/wq -> I8QL_ERR_ALIGN; k > 133144 -> I8QL_ERR_K_TOO_LARGE; other
 * y_dtype -> I8QL_ERR_DTYPE; bias with I32 -> I8QL_ERR_ARG.
 */
i8ql_status w8a8_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                      const float* w_scale, const float* bias, void* y, i8ql_dtype y_dtype,
                      int64_t m, int64_t n, int64_t k, void* stream);

/*
 * W8A8 plans: tile configurations, k split across workgroups, the workspace a split needs;
 * introspection and explicit selection, for tuning and for tests that cover every plan.
 *
 * A plan is one of I8QL_W8A8_NUM_CONFIGS tile configurations and a split count p: with
 * p > 1 the k steps of every output tile are divided between p workgroups, which store their
 * int32 partial tiles in a caller-provided workspace; the last of them to finish adds the
 * others' partials to its own and applies the epilogue.  int32 addition is exact, so every
 * plan computes bitwise the same outputs (exact accumulation, the same float32 epilogue) and
 * the choice affects only speed.  w8a8_gemm takes no workspace and launches the cost
 * model's best plan without a split; w8a8_gemm_with_plan launches the best plan whose
 * workspace fits in the one it is given (a model of the launch time on MI355X: rounds of
 * work units over the device's compute units, k steps per unit, the split's fix-up).
 *
 * Workspace contract: device memory, 16-byte aligned, zero-filled before its first use.
 * Its first 16 KiB are per-tile arrival counters (a split plan has at most
 * I8QL_W8A8_SPLIT_MAX_TILES output tiles), which every call returns to zero; the partial
 * tiles follow them.  So the same workspace serves any later call without clearing, as long
 * as nothing else writes its first 16 KiB.  Calls that may overlap in time (different
 * streams) must not share a workspace.
 *
 * w8a8_gemm_config_info(config, out5): writes {tile rows, tile columns, k-groups, 1 if k may
 *   be split across workgroups else 0, 1 if it runs w8a8_gemm_g128 else 0} of the
 *   configuration (host, 5 int32).  A configuration with g > 1 k-groups splits k inside the
 *   workgroup and accepts only k % (128 * g) == 0.
 *   Errors: out5 NULL -> I8QL_ERR_NULL; config outside [0, I8QL_W8A8_NUM_CONFIGS) ->
 *   I8QL_ERR_ARG.
 * w8a8_gemm_choose_config(m, n, k, cus): the configuration w8a8_gemm launches for an
 *   m x n x k product on a device with `cus` compute units (host arithmetic only, no HIP
 *   call); -1 if the sizes are not a valid non-empty w8a8_gemm call or cus < 1.
 * w8a8_gemm_with_config(config, ...): w8a8_gemm with the given configuration and no split
 *   (config == -1: the cost model's choice, exactly w8a8_gemm).  Arguments, results and
 *   errors as for w8a8_gemm, plus: config outside [-1, I8QL_W8A8_NUM_CONFIGS), or a
 *   configuration with g > 1 k-groups and k % (128 * g) != 0 -> I8QL_ERR_ARG.
 * w8a8_gemm_choose_plan(m, n, k, cus, workspace_bytes, out2): writes {config, splits} of the
 *   plan w8a8_gemm_with_plan(-1, -1, ...) launches with a workspace of workspace_bytes
 *   (host, 2 int32).  Errors: out2 NULL -> I8QL_ERR_NULL; invalid sizes, cus < 1 or
 *   workspace_bytes < 0 -> I8QL_ERR_ARG.
 * w8a8_gemm_workspace_size(config, splits, m, n, k, cus): the workspace bytes plan
 *   (config, splits) needs for an m x n x k product (0 without a split); with (-1, -1), those
 *   of the plan the cost model prefers on `cus` compute units with no limit on the
 *   workspace, which w8a8_gemm_with_plan(-1, -1, ...) then launches when given that much.
 *   -1 for invalid sizes or an invalid plan.
 * w8a8_gemm_with_plan(config, splits, ..., workspace, workspace_bytes, stream): w8a8_gemm
 *   with plan (config, splits), or with (-1, -1) the cost model's best plan whose workspace
 *   fits in workspace_bytes (workspace may be NULL with workspace_bytes 0: no split).
 *   workspace: device, workspace_bytes bytes, per the workspace contract above.
 *   Arguments, results and errors as for w8a8_gemm_with_config, plus: config == -1 with
 *   splits != -1, config >= 0 with splits outside [1, I8QL_W8A8_MAX_SPLITS], splits > 1 on a
 *   configuration that cannot split or with more splits than k steps of 128, or
 *   workspace_bytes < 0 -> I8QL_ERR_ARG; a split plan with more than
 *   I8QL_W8A8_SPLIT_MAX_TILES output tiles -> I8QL_ERR_SHAPE; the plan needs workspace but workspace is NULL ->
 *   I8QL_ERR_NULL; workspace not 16-byte aligned -> I8QL_ERR_ALIGN; workspace_bytes below
 *   what the plan needs -> I8QL_ERR_WORKSPACE.
 */
#define I8QL_W8A8_NUM_CONFIGS 12
#define I8QL_W8A8_MAX_SPLITS 8
#define I8QL_W8A8_SPLIT_MAX_TILES 4096
i8ql_status w8a8_gemm_config_info(int config, int32_t* out5);
int w8a8_gemm_choose_config(int64_t m, int64_t n, int64_t k, int cus);
i8ql_status w8a8_gemm_with_config(int config, const int8_t* xq, const float* x_scale,
                                  const int8_t* wq, const float* w_scale, const float* bias,
                                  void* y, i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                  void* stream);
i8ql_status w8a8_gemm_choose_plan(int64_t m, int64_t n, int64_t k, int cus,
                                  int64_t workspace_bytes, int32_t* out2);
int64_t w8a8_gemm_workspace_size(int config, int splits, int64_t m, int64_t n, int64_t k,
                                 int cus);

/*
 * w8a8_gemm_noalloc — w8a8_gemm_with_plan with the library's own workspace instead of a
 * caller's, for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The call allocates nothing.
 *
 * The workspace is a static device array of I8QL_W8A8_SCRATCH_BYTES, one copy per GPU,
 * held until the process ends.  Every call on a GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (other streams or host threads) race: the caller serializes
 * them.  The kernels return its arrival counters to zero after every call.  The first call
 * on a device looks up the array's address and clears its counters with one small kernel
 * on `stream`; make that first call outside graph capture.
 *
 * Plan (-1, -1): the cost model's best plan whose workspace fits in the array.  Arguments,
 * results and errors as for w8a8_gemm_with_plan without the workspace arguments, plus: an
 * explicit plan that needs more than I8QL_W8A8_SCRATCH_BYTES -> I8QL_ERR_WORKSPACE.
 */
#define I8QL_W8A8_SCRATCH_BYTES (32 * 1024 * 1024)
i8ql_status w8a8_gemm_noalloc(int config, int splits, const int8_t* xq, const float* x_scale,
                              const int8_t* wq, const float* w_scale, const float* bias, void* y,
                              i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                              void* stream);
i8ql_status w8a8_gemm_with_plan(int config, int splits, const int8_t* xq, const float* x_scale,
                                const int8_t* wq, const float* w_scale, const float* bias,
                                void* y, i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * w8a16_gemm — weight-only int8 GEMM for decode: int8 weights are dequantized in registers
 * and multiplied with 16-bit activations.
 *
 * Defines: [P5a] Summary (weight-only int8 saves memory bandwidth, not arithmetic);
 * [Day6] block 5 (W4A16-style weight-only: codes are expanded to bf16 inside the kernel,
 * the product runs at 16 bits, a pure bandwidth win that helps decode).
 *
 *   y[i, j] = w_scale[j] * sum_c x[i, c] * wq[j, c]  (+ bias[j])
 *   Each product of a bf16 value and an int8 code is exact; the sum is accumulated in
 *   float32 (its order is unspecified but fixed); stored as float32 or rne bfloat16.
 *
 * x        device, [m, k] bfloat16, 16-byte aligned.
 * wq       device, [n, k] int8, 16-byte aligned.   w_scale  device, [n] float32.
 * bias     device, [n] float32, or NULL.           y        device, [m, n] of y_dtype.
 * y_dtype in {I8QL_BF16, I8QL_F32}.  m, n >= 0; k >= 16, k % 16 == 0.  Any m is accepted;
 * the kernel is built for m <= 16 and stays correct (slower per row) above it.
 * Errors as for w8a8_gemm (no k upper limit: float32 accumulation).
 */
i8ql_status w8a16_gemm(const void* x, const int8_t* wq, const float* w_scale, const float* bias,
                       void* y, i8ql_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                       void* stream);

/*
 * grouped_w8a16_gemm — one launch of weight-only int8 GEMMs over routed experts, with the
 * expert-grouped dispatch done inside the kernel.
 *
 * Defines: [P5a] Summary (a grouped GEMM over all experts of a mixture-of-experts block with
 * per-output-channel int8 expert weights, stacked into one shared tensor per projection).
 *
 * Assignment p = i * topk + j (token i, routing slot j) uses expert e = expert_ids[i, j]:
 *   xrow(p)  = x[i, :]  when x_per_assignment == 0  (gate/up projections: token rows)
 *            = x[p, :]  when x_per_assignment == 1  (down projection: one row per assignment)
 *   if 0 <= e < num_experts:  y[p, c] = w_scale[e, c] * sum_d xrow(p)[d] * wq[e, c, d]
 *   else:                     y[p, :] = 0   (a caller-contract violation, made visible)
 *   float32 accumulation, stored as float32 or rne bfloat16.  Always-on shared experts are
 *   passed as extra experts appended to every token's id list.
 *
 * x           device, bfloat16, [t, k] (x_per_assignment == 0) or [t * topk, k] (== 1),
 *             16-byte aligned.
 * wq          device, [num_experts, n, k] int8, 16-byte aligned.
 * w_scale     device, [num_experts, n] float32.
 * expert_ids  device, [t, topk] int32.
 * y           device, [t * topk, n] of y_dtype in {I8QL_BF16, I8QL_F32}.
 * t, n >= 0; 1 <= topk <= 64; t * topk <= 65536; 1 <= num_experts <= 65534;
 * 16 <= k <= I8QL_GROUPED_MAX_K, k % 16 == 0 (an activation row is staged whole in LDS).
 * Errors: as for w8a16_gemm; x_per_assignment not 0/1, topk or num_experts out of range ->
 * I8QL_ERR_ARG; t * topk > 65536 or k > I8QL_GROUPED_MAX_K -> I8QL_ERR_SHAPE.
 */
#define I8QL_GROUPED_MAX_K 32768
i8ql_status grouped_w8a16_gemm(const void* x, int x_per_assignment, const int8_t* wq,
                               const float* w_scale, int64_t num_experts,
                               const int32_t* expert_ids, int64_t t, int64_t topk, void* y,
                               i8ql_dtype y_dtype, int64_t n, int64_t k, void* stream);

/*
 * One scale per group of I8QL_GROUP_SIZE input channels.  Defines: [Day6] The mechanism,
 * block 1 (a scale can cover a tensor, a row, or a run of 128 consecutive input channels;
 * an outlier then coarsens only the codes of its own run).
 */
#define I8QL_GROUP_SIZE 128

/*
 * quantize_per_group_int8 — the quantize_per_channel_int8 rule (float32 absmax / 127,
 * correctly rounded float32 quotient, round half to even, clamp to [-127, 127], all-zero
 * group -> scale 1 and codes 0) applied to every group of 128 consecutive elements of a row.
 *
 * w          device, [n, k] of w_dtype in {I8QL_F32, I8QL_BF16, I8QL_F16}, 16-byte aligned.
 * q_out      device, [n, k] int8, 8-byte aligned.
 * scale_out  device, [n, k / 128] float32 (group g of row i at i * (k / 128) + g).
 * n >= 0, k >= 128, k % 128 == 0.
 * Errors: dtype -> I8QL_ERR_DTYPE; n < 0 or k not a positive multiple of 128 ->
 * I8QL_ERR_SHAPE; NULL -> I8QL_ERR_NULL; alignment -> I8QL_ERR_ALIGN.
 */
i8ql_status quantize_per_group_int8(const void* w, i8ql_dtype w_dtype, int64_t n, int64_t k,
                                    int8_t* q_out, float* scale_out, void* stream);

/*
 * w8a16_gemm_g128 — w8a16_gemm with group scales:
 *   y[i, j] = sum_g w_scale[j, g] * sum_{c in group g} x[i, c] * wq[j, c]  (+ bias[j])
 * with float32 partial sums per group.  Arguments as for w8a16_gemm except
 * w_scale [n, k / 128] float32 (from quantize_per_group_int8) and k % 128 == 0
 * (I8QL_ERR_SHAPE otherwise).
 */
i8ql_status w8a16_gemm_g128(const void* x, const int8_t* wq, const float* w_scale,
                            const float* bias, void* y, i8ql_dtype y_dtype, int64_t m,
                            int64_t n, int64_t k, void* stream);

/*
 * w8a8_gemm_g128 — W8A8 with one weight scale per group of I8QL_GROUP_SIZE input channels.
 *
 * Defines: [Day6] The mechanism, block 1 (a weight scale per run of 128 consecutive input
 * channels, so an outlier coarsens only its own run) and block 5 (both operands int8, the
 * product on the 8-bit matrix units); per-token activation scales as for w8a8_gemm.
 *
 *   part_g[i, j] = sum_{c in group g} xq[i, c] * wq[j, c]          (exact, int32)
 *   y[i, j]      = x_scale[i] * sum_g w_scale[j, g] * part_g[i, j]  (+ bias[j])
 *   in float32: each group's partial is converted (exactly) and multiplied by its scale with
 *   one rounding into a running sum, in increasing g; the sum is then multiplied by
 *   x_scale[i] and the bias added (round to nearest each); stored as float32 or rne bfloat16.
 *
 * xq [m, k] and wq [n, k] int8, 16-byte aligned; x_scale [m] float32; w_scale [n, k / 128]
 * float32 (as quantize_per_group_int8 writes it); bias [n] float32 or NULL; y [m, n] of
 * y_dtype in {I8QL_BF16, I8QL_F32}.  m, n >= 0; k >= 128, k % 128 == 0.
 * Errors: y_dtype I32 or another dtype -> I8QL_ERR_DTYPE (the int32 accumulator of all groups
 * is w8a8_gemm's); k not a positive multiple of 128 or too many tiles -> I8QL_ERR_SHAPE;
 * NULL -> I8QL_ERR_NULL; alignment -> I8QL_ERR_ALIGN.
 * w8a8_gemm_g128_with_config(config, ...): on configuration `config`, which must run group
 * scales (w8a8_gemm_config_info), or -1 for the cost model's choice; other values ->
 * I8QL_ERR_ARG.
 */
i8ql_status w8a8_gemm_g128(const int8_t* xq, const float* x_scale, const int8_t* wq,
                           const float* w_scale, const float* bias, void* y, i8ql_dtype y_dtype,
                           int64_t m, int64_t n, int64_t k, void* stream);
i8ql_status w8a8_gemm_g128_with_config(int config, const int8_t* xq, const float* x_scale,
                                       const int8_t* wq, const float* w_scale,
                                       const float* bias, void* y, i8ql_dtype y_dtype,
                                       int64_t m, int64_t n, int64_t k, void* stream);

/*
 * The mixture-of-experts steps on either side of grouped_w8a16_gemm.  [P5a] Summary runs the
 * grouped GEMM inside the mixture-of-experts block of deepseek-moe-16b but does not spell out
 * the block's routing, activation or combine; these entry points take the plainest reading
 * (softmax top-k routing with unrenormalized weights and shared experts appended; SiLU·mul
 * between the gate/up and down projections; a routing-weighted sum of each token's rows).
 */

#define I8QL_ROUTE_MAX_EXPERTS 256
#define I8QL_ROUTE_MAX_K 32

/*
 * moe_route_topk — top-k routing from router logits.
 *
 * For token i: p = softmax(logits[i, :]) over the e_routed routed experts; slots
 * 0 .. k_routed - 1 hold the k_routed experts with the largest logits in decreasing order
 * (equal logits: lower expert index first) with weights p of those experts (not
 * renormalized); slots k_routed .. k_routed + n_shared - 1 hold the shared experts
 * e_routed .. e_routed + n_shared - 1 with weight 1.  The ids feed grouped_w8a16_gemm (with
 * num_experts = e_routed + n_shared) and the weights moe_combine.  Float32 arithmetic; the
 * ids are decided by exact comparisons of the logits.
 *
 * logits   device, [t, e_routed] of logits_dtype in {I8QL_F32, I8QL_BF16}; finite values.
 * ids      device, [t, k_routed + n_shared] int32.
 * weights  device, [t, k_routed + n_shared] float32.
 * 1 <= e_routed <= I8QL_ROUTE_MAX_EXPERTS; 1 <= k_routed <= min(e_routed, I8QL_ROUTE_MAX_K);
 * 0 <= n_shared <= I8QL_ROUTE_MAX_K; k_routed + n_shared <= 64; t >= 0.
 * Errors: dtype -> I8QL_ERR_DTYPE; t < 0 -> I8QL_ERR_SHAPE; the expert counts out of range
 * -> I8QL_ERR_ARG; NULL -> I8QL_ERR_NULL; misaligned element pointers -> I8QL_ERR_ALIGN.
 */
i8ql_status moe_route_topk(const void* logits, i8ql_dtype logits_dtype, int64_t t,
                           int64_t e_routed, int64_t k_routed, int64_t n_shared, int32_t* ids,
                           float* weights, void* stream);

/*
 * grouped_w8a16_silu_gemm — the gate and up projections of the experts as one grouped
 * weight-only GEMM with the SiLU·mul fused into its epilogue.
 *
 * Each expert's weights are stacked [2n, k]: rows 0 .. n-1 are the gate projection, rows
 * n .. 2n-1 the up projection (w_scale likewise [num_experts, 2n]).  For assignment p routed
 * to a valid expert: g = grouped_w8a16_gemm's value of gate row c, u = that of up row c,
 * h[p, c] = g / (1 + exp(-g)) * u (float32), stored as float32 or rne bfloat16; rows of
 * invalid ids are 0.  Everything else (x, x_per_assignment, expert_ids, t, topk, k, limits,
 * errors) as for grouped_w8a16_gemm, with wq [num_experts, 2n, k] and h [t * topk, n].
 */
i8ql_status grouped_w8a16_silu_gemm(const void* x, int x_per_assignment, const int8_t* wq,
                                    const float* w_scale, int64_t num_experts,
                                    const int32_t* expert_ids, int64_t t, int64_t topk, void* h,
                                    i8ql_dtype h_dtype, int64_t n, int64_t k, void* stream);

/*
 * moe_combine — the routing-weighted sum of each token's assignment rows:
 *   y[i, c] = sum_j weights[i, j] * d[i * topk + j, c],  j = 0 .. topk-1 in order, float32.
 *
 * d        device, [t * topk, n] of d_dtype in {I8QL_BF16, I8QL_F32} (e.g. the down
 *          projection's grouped_w8a16_gemm output).
 * weights  device, [t, topk] float32 (e.g. from moe_route_topk).
 * y        device, [t, n] of y_dtype in {I8QL_BF16, I8QL_F32}; must not alias d.
 * 1 <= topk <= 64; t, n >= 0.  Rows that are 16-byte aligned whole chunks take 16-byte
 * accesses, any other layout the element path.
 * Errors: dtype -> I8QL_ERR_DTYPE; topk -> I8QL_ERR_ARG; negative or too large t, n ->
 * I8QL_ERR_SHAPE; NULL -> I8QL_ERR_NULL; misaligned element pointers -> I8QL_ERR_ALIGN.
 */
i8ql_status moe_combine(const void* d, i8ql_dtype d_dtype, const float* weights, int64_t t,
                        int64_t topk, int64_t n, void* y, i8ql_dtype y_dtype, void* stream);

/* Host: a static, human-readable name for a status code ("I8QL_OK", ...). */
const char* i8ql_status_string(i8ql_status s);

/* Host: the hipError_t (as int) recorded by the most recent call on this thread that
 * returned I8QL_ERR_HIP, or 0. */
int i8ql_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* I8QL_H */
