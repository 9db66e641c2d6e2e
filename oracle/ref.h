/*
 * ref.h — CPU oracle of the int8 quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load or call it.  It shares no code, header, table or helper with the
 * HIP library and includes nothing from it.
 *
 * Pages followed (cited by title and section):
 *   [P5a]  "Phase 5a: int8 weight-only quantization", Summary.
 *   [W8A8] "feat(quantization): support compressed-tensors W8A8 and mixed modules",
 *          "Design and Supported Execution Scheme".
 *   [Day6] "Day 6 — Quantize It Yourself", "The mechanism", blocks 1 and 5.
 */
#ifndef I8QL_ORACLE_REF_H
#define I8QL_ORACLE_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input element codes understood by ref_quantize_rows. */
enum { REF_F32 = 0, REF_BF16 = 1, REF_F16 = 2 };

void ref_set_threads(int n);
int ref_get_threads(void);

/* Row quantizer: [Day6] block 1, [P5a] Summary (float32 arithmetic, all-zero guard).
 * a: [r, k] of dtype; q: [r, k]; s: [r].  Returns 0, or -1 on a bad dtype. */
int ref_quantize_rows(const void* a, int dtype, int64_t r, int64_t k, int8_t* q, float* s);

/* W8A8: [W8A8] design section, [Day6] block 5.  acc: [m, n] exact int32 sums; y: [m, n]
 * epilogue value acc * x_scale[i] * w_scale[j] (+ bias[j]) in double (may be NULL).
 * bias may be NULL.  Returns 0, or -1 when some sum does not fit in int32. */
int ref_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
             const float* bias, int64_t m, int64_t n, int64_t k, int32_t* acc, double* y);

/* W8A16: [P5a] Summary, [Day6] block 5.  x: [m, k] bfloat16 bit patterns; y: [m, n] double
 * value w_scale[j] * sum_c x[i, c] * wq[j, c] (+ bias[j]). */
void ref_w8a16(const uint16_t* x, const int8_t* wq, const float* w_scale, const float* bias,
               int64_t m, int64_t n, int64_t k, double* y);

/* Grouped W8A16 over routed experts: [P5a] Summary.  x: [t, k] (x_per_assignment == 0) or
 * [t * topk, k] bfloat16 bits; wq: [e, n, k]; w_scale: [e, n]; ids: [t, topk];
 * y: [t * topk, n] double; rows whose id is outside [0, e) are zero. */
void ref_grouped_w8a16(const uint16_t* x, int x_per_assignment, const int8_t* wq,
                       const float* w_scale, int64_t e, const int32_t* ids, int64_t t,
                       int64_t topk, int64_t n, int64_t k, double* y);

/* One scale per group of `group` input channels ([Day6] block 1): the row rule per group.
 * q: [r, k]; s: [r, k / group].  Returns 0, or -1 on a bad dtype or k % group != 0. */
int ref_quantize_groups(const void* a, int dtype, int64_t r, int64_t k, int64_t group, int8_t* q,
                        float* s);
/* W8A16 with group scales w_scale [n, k / group]: y [m, n] double. */
void ref_w8a16_grouped_scales(const uint16_t* x, const int8_t* wq, const float* w_scale,
                              const float* bias, int64_t m, int64_t n, int64_t k, int64_t group,
                              double* y);

/* W8A8 with group weight scales w_scale [n, k / group] ([Day6] blocks 1 and 5): y [m, n]
 * double = x_scale[i] * sum_g w_scale[j, g] * (exact int sum of group g) (+ bias[j]). */
void ref_w8a8_grouped_scales(const int8_t* xq, const float* x_scale, const int8_t* wq,
                             const float* w_scale, const float* bias, int64_t m, int64_t n,
                             int64_t k, int64_t group, double* y);

/* Mixture-of-experts steps around the grouped GEMM ([P5a] Summary names the block; its
 * routing, activation and combine are readings, stated in ref.c). */
void ref_moe_route_topk(const float* logits, int64_t t, int64_t e_routed, int64_t k_routed,
                        int64_t n_shared, int32_t* ids, double* w);
void ref_grouped_w8a16_silu(const uint16_t* x, int x_per_assignment, const int8_t* wq,
                            const float* w_scale, int64_t e, const int32_t* ids, int64_t t,
                            int64_t topk, int64_t n, int64_t k, double* h);
void ref_moe_combine(const float* d, const float* w, int64_t t, int64_t topk, int64_t n,
                     double* y);

/* RMS normalization (optional residual add) of bf16 rows, output bf16: the producer of a
 * decoder layer's quantized inputs.  The norm is not on the pages; its reading is stated in
 * ref.c.  residual and res_out may be NULL (both or neither). */
void ref_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma, float eps,
                 int64_t m, int64_t k, uint16_t* res_out, uint16_t* h);

/* SiLU·mul of a gate/up product [m, 2i] bf16 (gate columns first), rounded to bf16 h [m, i];
 * optionally the bf16 on the other side of each exact value and a flag where the exact value
 * is within rel of the halfway point (reading stated in ref.c). */
void ref_silu_mul(const uint16_t* gu, int64_t m, int64_t i, double rel, uint16_t* h,
                  uint16_t* other, uint8_t* amb);
/* The row quantizer's code step under given scales: clamp(rne(fl32(a / s)), -127, 127). */
void ref_codes_with_scale(const uint16_t* a, const float* s, int64_t r, int64_t k, int8_t* q);

#ifdef __cplusplus
}
#endif
#endif
