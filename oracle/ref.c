/*
 * ref.c — CPU oracle of the int8 quantized linear layer: plain loops, written from the pages.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load or call it.  It shares no code with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.  Float32 work is
 * IEEE binary32 with round to nearest even and no flush-to-zero (x86-64 SSE defaults).
 * OpenMP only splits independent output rows across threads; it changes no arithmetic.
 *
 * Mutants (teeth for the pins; never built into the normal library):
 *   -DREF_MUTANT_BF16_ARITH  do the quantizer arithmetic in bfloat16, the first precision
 *                            bug that "Phase 5a: int8 weight-only quantization" (Summary)
 *                            reports;
 *   -DREF_MUTANT_FLOOR_SCALE floor every small scale at a dtype-dependent minimum, the
 *                            second bug that the same Summary reports.
 */
#include "ref.h"

#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

void ref_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int ref_get_threads(void) { return omp_get_max_threads(); }

/* ---- exact widening of the input formats to float32 ---------------------------------- */

static float bf16_to_f32(uint16_t b) {
  /* bfloat16 is the upper half of a binary32 word. */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static float f16_to_f32(uint16_t h) {
  /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  float mag;
  if (e == 0)
    mag = ldexpf((float)f, -24); /* subnormal: f * 2^-24 */
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexpf((float)(f | 0x400), e - 25); /* (1024 + f) * 2^(e - 25) */
  return sign ? -mag : mag;
}

static float load_elem(const void* a, int dtype, int64_t i) {
  switch (dtype) {
    case REF_F32: return ((const float*)a)[i];
    case REF_BF16: return bf16_to_f32(((const uint16_t*)a)[i]);
    default: return f16_to_f32(((const uint16_t*)a)[i]);
  }
}

/* ---- the quantizer ---------------------------------------------------------------------- */

/* Round to the nearest integer, ties to the even one.  |t| < 2^23, so t - floor(t) is exact. */
static float round_half_even(float t) {
  float f = floorf(t);
  float d = t - f;
  if (d > 0.5f) return f + 1.0f;
  if (d < 0.5f) return f;
  return (fmodf(f, 2.0f) == 0.0f) ? f : f + 1.0f;
}

#ifdef REF_MUTANT_BF16_ARITH
/* Round a float32 to the nearest bfloat16 (ties to even), kept as float32. */
static float to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  uint32_t lsb = (u >> 16) & 1u;
  u = (u + 0x7fffu + lsb) & 0xffff0000u;
  memcpy(&x, &u, sizeof x);
  return x;
}
#endif

/*
 * One scale per row, the symmetric absmax rule of "Day 6 — Quantize It Yourself" (The
 * mechanism, block 1): s = absmax / largest code, q = clamp(round(w / s)).  The grid is
 * symmetric, so the largest code is 127 and -128 is never used.  "Phase 5a: int8
 * weight-only quantization" (Summary, bug fixes) fixes two details: every step is float32
 * arithmetic, whatever the weight's own dtype, and the guard against 0/0 applies only to a
 * channel whose scale is zero; its stored scale is 1 and its codes are 0.
 */
int ref_quantize_rows(const void* a, int dtype, int64_t r, int64_t k, int8_t* q, float* s) {
  if (dtype != REF_F32 && dtype != REF_BF16 && dtype != REF_F16) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < r; ++row) {
    const int64_t base = row * k;
    float amax = 0.0f;
    for (int64_t j = 0; j < k; ++j) {
      float v = fabsf(load_elem(a, dtype, base + j));
      if (v > amax) amax = v;
    }
    float scale = amax / 127.0f;
#ifdef REF_MUTANT_BF16_ARITH
    if (dtype != REF_F32) scale = to_bf16(scale);
#endif
#ifdef REF_MUTANT_FLOOR_SCALE
    {
      /* smallest normal number of the input format, divided by the largest code */
      float floor_v = (dtype == REF_F16) ? ldexpf(1.0f, -14) / 127.0f
                                          : ldexpf(1.0f, -126) / 127.0f;
      if (scale < floor_v) scale = floor_v;
    }
#endif
    if (scale == 0.0f) {
      s[row] = 1.0f;
      for (int64_t j = 0; j < k; ++j) q[base + j] = 0;
      continue;
    }
    for (int64_t j = 0; j < k; ++j) {
      float t = load_elem(a, dtype, base + j) / scale;
#ifdef REF_MUTANT_BF16_ARITH
      if (dtype != REF_F32) t = to_bf16(t);
#endif
      float c = round_half_even(t);
      if (c > 127.0f) c = 127.0f;
      if (c < -127.0f) c = -127.0f;
      q[base + j] = (int8_t)c;
    }
    s[row] = scale;
  }
  return 0;
}

/* ---- W8A8 ------------------------------------------------------------------------------- */

/*
 * int8 x int8 products summed exactly, then the per-token scale, the per-channel scale and
 * the bias ("feat(quantization): support compressed-tensors W8A8 and mixed modules", Design
 * and Supported Execution Scheme: per-channel weights, per-token activations, no output
 * quantization).  The sum is formed in int64 and checked against the int32 range.
 */
int ref_w8a8(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
             const float* bias, int64_t m, int64_t n, int64_t k, int32_t* acc, double* y) {
  int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
  for (int64_t i = 0; i < m; ++i) {
    const int8_t* xr = xq + i * k;
    for (int64_t j = 0; j < n; ++j) {
      const int8_t* wr = wq + j * k;
      int64_t sum = 0;
      for (int64_t c = 0; c < k; ++c) sum += (int64_t)xr[c] * (int64_t)wr[c];
      if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
      acc[i * n + j] = (int32_t)sum;
      if (y) {
        double v = (double)sum * (double)x_scale[i] * (double)w_scale[j];
        if (bias) v += (double)bias[j];
        y[i * n + j] = v;
      }
    }
  }
  return overflow ? -1 : 0;
}

/* ---- W8A16 ------------------------------------------------------------------------------ */

/*
 * Weight-only: y = x * dequant(W)^T with dequant(W)[j, c] = w_scale[j] * wq[j, c]
 * ("Phase 5a: int8 weight-only quantization", Summary; "Day 6 — Quantize It Yourself", The
 * mechanism, block 5).  Each bf16 * int8 product is exact in double; the sum is double.
 */
void ref_w8a16(const uint16_t* x, const int8_t* wq, const float* w_scale, const float* bias,
               int64_t m, int64_t n, int64_t k, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    const uint16_t* xr = x + i * k;
    for (int64_t j = 0; j < n; ++j) {
      const int8_t* wr = wq + j * k;
      double sum = 0.0;
      for (int64_t c = 0; c < k; ++c) sum += (double)bf16_to_f32(xr[c]) * (double)wr[c];
      double v = (double)w_scale[j] * sum;
      if (bias) v += (double)bias[j];
      y[i * n + j] = v;
    }
  }
}

/* ---- grouped W8A16 ---------------------------------------------------------------------- */

/*
 * Grouped GEMM over routed experts ("Phase 5a: int8 weight-only quantization", Summary):
 * assignment p = (token i, slot j) multiplies its input row by the stacked weights of expert
 * ids[i, j].  An id outside [0, e) yields a zero row.
 */
void ref_grouped_w8a16(const uint16_t* x, int x_per_assignment, const int8_t* wq,
                       const float* w_scale, int64_t e, const int32_t* ids, int64_t t,
                       int64_t topk, int64_t n, int64_t k, double* y) {
  const int64_t rows = t * topk;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < rows; ++p) {
    const int64_t tok = p / topk;
    const int32_t ex = ids[p];
    const uint16_t* xr = x + (x_per_assignment ? p : tok) * k;
    for (int64_t j = 0; j < n; ++j) {
      if (ex < 0 || ex >= e) {
        y[p * n + j] = 0.0;
        continue;
      }
      const int8_t* wr = wq + ((int64_t)ex * n + j) * k;
      double sum = 0.0;
      for (int64_t c = 0; c < k; ++c) sum += (double)bf16_to_f32(xr[c]) * (double)wr[c];
      y[p * n + j] = (double)w_scale[(int64_t)ex * n + j] * sum;
    }
  }
}

/* ---- the steps around the grouped GEMM in a mixture-of-experts block ------------------- */

/*
 * "Phase 5a: int8 weight-only quantization" (Summary) measures the grouped GEMM inside the
 * mixture-of-experts block of deepseek-moe-16b, but no page spells out the block's other
 * steps.  The three functions below take the plainest reading that the rest supports:
 *   routing  — softmax over the routed experts' logits; the k_routed largest probabilities
 *              (equivalently logits) are kept, unrenormalized, as the routing weights; equal
 *              logits go to the lower expert index first; the always-on shared experts are
 *              appended after them (ids e_routed .. e_routed + n_shared - 1, weight 1);
 *   SiLU·mul — between the gate/up projections and the down projection,
 *              h = silu(gate) * up with silu(v) = v / (1 + exp(-v));
 *   combine  — each token's output is the routing-weighted sum of its assignments' rows.
 * Everything is computed in double.
 */

/* Routing.  logits: [t, e_routed] float32; ids: [t, k_routed + n_shared]; w: same, double.
 * Slots hold the selected experts by decreasing logit (ties: lower index first). */
void ref_moe_route_topk(const float* logits, int64_t t, int64_t e_routed, int64_t k_routed,
                        int64_t n_shared, int32_t* ids, double* w) {
  const int64_t kk = k_routed + n_shared;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < t; ++i) {
    const float* l = logits + i * e_routed;
    double mx = -INFINITY;
    for (int64_t j = 0; j < e_routed; ++j)
      if ((double)l[j] > mx) mx = (double)l[j];
    double den = 0.0;
    for (int64_t j = 0; j < e_routed; ++j) den += exp((double)l[j] - mx);
    /* selection: k_routed times, the largest logit not taken yet (first index on ties) */
    for (int64_t s = 0; s < k_routed; ++s) {
      int64_t best = -1;
      for (int64_t j = 0; j < e_routed; ++j) {
        int taken = 0;
        for (int64_t u = 0; u < s; ++u)
          if (ids[i * kk + u] == (int32_t)j) taken = 1;
        if (taken) continue;
        if (best < 0 || l[j] > l[best]) best = j;
      }
      ids[i * kk + s] = (int32_t)best;
      w[i * kk + s] = exp((double)l[best] - mx) / den;
    }
    for (int64_t s = 0; s < n_shared; ++s) {
      ids[i * kk + k_routed + s] = (int32_t)(e_routed + s);
      w[i * kk + k_routed + s] = 1.0;
    }
  }
}

/* SiLU·mul after a grouped gate/up product: wq is [e, 2n, k] with the gate rows of each
 * expert first and its up rows after them, w_scale [e, 2n].  h: [t * topk, n] double,
 * h = silu(gate) * up of the exact double products (zero rows for invalid ids). */
void ref_grouped_w8a16_silu(const uint16_t* x, int x_per_assignment, const int8_t* wq,
                            const float* w_scale, int64_t e, const int32_t* ids, int64_t t,
                            int64_t topk, int64_t n, int64_t k, double* h) {
  const int64_t rows = t * topk;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < rows; ++p) {
    const int64_t tok = p / topk;
    const int32_t ex = ids[p];
    const uint16_t* xr = x + (x_per_assignment ? p : tok) * k;
    for (int64_t j = 0; j < n; ++j) {
      if (ex < 0 || ex >= e) {
        h[p * n + j] = 0.0;
        continue;
      }
      const int8_t* wg = wq + ((int64_t)ex * 2 * n + j) * k;
      const int8_t* wu = wq + ((int64_t)ex * 2 * n + n + j) * k;
      double sg = 0.0, su = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        const double xv = (double)bf16_to_f32(xr[c]);
        sg += xv * (double)wg[c];
        su += xv * (double)wu[c];
      }
      const double g = (double)w_scale[(int64_t)ex * 2 * n + j] * sg;
      const double u = (double)w_scale[(int64_t)ex * 2 * n + n + j] * su;
      h[p * n + j] = g / (1.0 + exp(-g)) * u;
    }
  }
}

/* Combine: y[i, c] = sum_j w[i, j] * d[i * topk + j, c].  d: [t * topk, n] float32 values;
 * w: [t, topk]; y: [t, n] double. */
void ref_moe_combine(const float* d, const float* w, int64_t t, int64_t topk, int64_t n,
                     double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < t; ++i)
    for (int64_t c = 0; c < n; ++c) {
      double acc = 0.0;
      for (int64_t j = 0; j < topk; ++j)
        acc += (double)w[i * topk + j] * (double)d[(i * topk + j) * n + c];
      y[i * n + c] = acc;
    }
}

/* ---- one scale per group of input channels --------------------------------------------- */

/*
 * "Day 6 — Quantize It Yourself", The mechanism, block 1: the scale may be shared by a
 * whole tensor, by one row (output channel), or by a run of 128 consecutive elements of a
 * row (input channels).  Each group of `group` consecutive elements of a row gets the row
 * quantizer's rule (float32 absmax / 127, float32 quotient, round half to even, clamp, the
 * all-zero guard).  q: [r, k]; s: [r, k / group], k % group == 0.
 */
int ref_quantize_groups(const void* a, int dtype, int64_t r, int64_t k, int64_t group, int8_t* q,
                        float* s) {
  if (dtype != REF_F32 && dtype != REF_BF16 && dtype != REF_F16) return -1;
  if (group < 1 || k % group != 0) return -1;
  const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < r; ++row) {
    for (int64_t g = 0; g < ng; ++g) {
      const int64_t base = row * k + g * group;
      float amax = 0.0f;
      for (int64_t j = 0; j < group; ++j) {
        float v = fabsf(load_elem(a, dtype, base + j));
        if (v > amax) amax = v;
      }
      const float scale = amax / 127.0f;
      if (scale == 0.0f) {
        s[row * ng + g] = 1.0f;
        for (int64_t j = 0; j < group; ++j) q[base + j] = 0;
        continue;
      }
      for (int64_t j = 0; j < group; ++j) {
        float c = round_half_even(load_elem(a, dtype, base + j) / scale);
        if (c > 127.0f) c = 127.0f;
        if (c < -127.0f) c = -127.0f;
        q[base + j] = (int8_t)c;
      }
      s[row * ng + g] = scale;
    }
  }
  return 0;
}

/* Weight-only product with one weight scale per (output channel, group of input channels):
 * y[i, j] = sum_g w_scale[j, g] * sum_{c in g} x[i, c] * wq[j, c] (+ bias[j]), in double. */
void ref_w8a16_grouped_scales(const uint16_t* x, const int8_t* wq, const float* w_scale,
                              const float* bias, int64_t m, int64_t n, int64_t k, int64_t group,
                              double* y) {
  const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    const uint16_t* xr = x + i * k;
    for (int64_t j = 0; j < n; ++j) {
      const int8_t* wr = wq + j * k;
      double v = 0.0;
      for (int64_t g = 0; g < ng; ++g) {
        double part = 0.0;
        for (int64_t c = g * group; c < (g + 1) * group; ++c)
          part += (double)bf16_to_f32(xr[c]) * (double)wr[c];
        v += (double)w_scale[j * ng + g] * part;
      }
      if (bias) v += (double)bias[j];
      y[i * n + j] = v;
    }
  }
}

/*
 * W8A8 with one weight scale per (output channel, group of `group` input channels): both
 * operands int8 ("Day 6 — Quantize It Yourself", The mechanism, block 5), the weight scale
 * shared by a run of consecutive input channels (same page, block 1), per-token activation
 * scales ("feat(quantization): support compressed-tensors W8A8 and mixed modules", Design and
 * Supported Execution Scheme).  Each group's code products are summed exactly (int64), the
 * group sums are weighted by their scales and added in double, then the token's scale and
 * the bias apply:
 *   y[i, j] = x_scale[i] * sum_g w_scale[j, g] * sum_{c in g} xq[i, c] * wq[j, c] (+ bias[j])
 */
void ref_w8a8_grouped_scales(const int8_t* xq, const float* x_scale, const int8_t* wq,
                             const float* w_scale, const float* bias, int64_t m, int64_t n,
                             int64_t k, int64_t group, double* y) {
  const int64_t ng = k / group;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    const int8_t* xr = xq + i * k;
    for (int64_t j = 0; j < n; ++j) {
      const int8_t* wr = wq + j * k;
      double v = 0.0;
      for (int64_t g = 0; g < ng; ++g) {
        int64_t part = 0;
        for (int64_t c = g * group; c < (g + 1) * group; ++c)
          part += (int64_t)xr[c] * (int64_t)wr[c];
        v += (double)w_scale[j * ng + g] * (double)part;
      }
      v *= (double)x_scale[i];
      if (bias) v += (double)bias[j];
      y[i * n + j] = v;
    }
  }
}

/* ---- the norm that produces a projection's input ------------------------------------- */

/* Round a float32 to the nearest bfloat16, ties to the one whose last bit is zero (finite
 * inputs; the result keeps the upper 16 bits). */
static uint16_t f32_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  const uint32_t low = u & 0xffffu;
  uint32_t hi = u >> 16;
  if (low > 0x8000u || (low == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/*
 * RMS normalization of bfloat16 rows, the step whose output a decoder layer quantizes per
 * token before its q/k/v and gate/up products (dynamic per-token activation quantization:
 * "feat(quantization): support compressed-tensors W8A8 and mixed modules", Design and
 * Supported Execution Scheme, and its Weight footprint section, where normalization
 * weights stay in higher precision; "Day 6 — Quantize It Yourself", Reading-share post,
 * fact 2, on the forward-pass work that per-token quantization adds).  No page writes the
 * norm out; the reading here:
 *   u = x, or with a residual stream u = bf16(x + residual) (one float32 addition), which is
 *       also the updated residual;
 *   S = sum over the row of u^2, in double;  v = fl32(S / k);
 *   r = fl32(1 / fl32(sqrt(fl32(v + eps))))  (three correctly rounded float32 operations);
 *   h = bf16(fl32(fl32(u * r) * gamma)).
 * x, residual: [m, k] bf16 bits (residual may be NULL); gamma: [k] bf16 bits;
 * res_out: [m, k] (NULL when residual is NULL); h: [m, k] bf16 bits.
 */
void ref_rmsnorm(const uint16_t* x, const uint16_t* residual, const uint16_t* gamma, float eps,
                 int64_t m, int64_t k, uint16_t* res_out, uint16_t* h) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    const int64_t base = i * k;
    double sum_sq = 0.0;
    for (int64_t c = 0; c < k; ++c) {
      float u = bf16_to_f32(x[base + c]);
      if (residual) {
        const uint16_t ub = f32_to_bf16_bits(u + bf16_to_f32(residual[base + c]));
        res_out[base + c] = ub;
        u = bf16_to_f32(ub);
      }
      sum_sq += (double)u * (double)u;
    }
    const float v = (float)(sum_sq / (double)k);
    const float r = 1.0f / sqrtf(v + eps);
    for (int64_t c = 0; c < k; ++c) {
      const float u = bf16_to_f32(residual ? res_out[base + c] : x[base + c]);
      const float t = u * r;
      h[base + c] = f32_to_bf16_bits(t * bf16_to_f32(gamma[c]));
    }
  }
}

/* ---- SiLU·mul that produces the down projection's input --------------------------------- */

/* The two bfloat16 values around a finite double v and whether v is within `rel` (relative)
 * of the point halfway between them.  near: the bf16 nearest to v (ties to even); other: the
 * neighbour on the other side of v (equal to near when v is a bf16 value).  Every bf16 value
 * is a double, and so is every halfway point, so the comparisons are exact. */
static void bf16_neighbours(double v, double rel, uint16_t* near, uint16_t* other, int* amb) {
  /* the float nearest to v lies within half a float ulp of v, so the bf16 values that
   * bracket v are the truncation of that float toward zero and the next one away from zero
   * (or the truncation and the previous one when the float sits on a bf16 value) */
  const float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint32_t lo_bits = u & 0xffff0000u; /* toward zero */
  float lo_f;
  memcpy(&lo_f, &lo_bits, sizeof lo_f);
  uint32_t hi_bits = lo_bits + 0x10000u; /* away from zero (same sign) */
  float hi_f;
  memcpy(&hi_f, &hi_bits, sizeof hi_f);
  if ((u & 0xffffu) == 0 && fabs((double)lo_f) > fabs(v)) {
    /* f is a bf16 value above |v|: the bracket is (previous, f) */
    hi_bits = lo_bits;
    hi_f = lo_f;
    lo_bits = lo_bits - 0x10000u;
    memcpy(&lo_f, &lo_bits, sizeof lo_f);
  }
  const double a = fabs(v), l = fabs((double)lo_f), h = fabs((double)hi_f);
  const double mid = 0.5 * (l + h); /* exact: l and h differ in the 8th significant bit */
  uint16_t pick, alt;
  if (a == l) {
    pick = (uint16_t)(lo_bits >> 16);
    alt = pick;
  } else if (a < mid || (a == mid && ((lo_bits >> 16) & 1u) == 0)) {
    pick = (uint16_t)(lo_bits >> 16);
    alt = (uint16_t)(hi_bits >> 16);
  } else {
    pick = (uint16_t)(hi_bits >> 16);
    alt = (uint16_t)(lo_bits >> 16);
  }
  *near = pick;
  *other = alt;
  *amb = (a != l) && fabs(a - mid) <= rel * a;
}

/*
 * SiLU·mul of a gate/up product, the step between a decoder MLP's gate/up projection and its
 * down projection (the same activation as the mixture-of-experts block's, reading stated
 * with ref_grouped_w8a16_silu; no page writes it out), written as the bf16 tensor that the
 * down projection's per-token quantization reads: h = silu(g) * u = g / (1 + e^(-g)) * u in
 * double, rounded to the nearest bf16 (ties to even).
 * gu: [m, 2 i] bf16 bits, the gate values in columns [0, i) and the up values in [i, 2 i)
 * (one GEMM over the stacked gate and up weights); h: [m, i] bf16 bits.  With `other` and
 * `amb` (both or neither NULL): the bf16 on the other side of the exact value, and 1 where
 * the exact value lies within `rel` (relative) of the halfway point between the two, i.e.
 * where a float32 evaluation of the same formula may round to either.
 */
void ref_silu_mul(const uint16_t* gu, int64_t m, int64_t i, double rel, uint16_t* h,
                  uint16_t* other, uint8_t* amb) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < m; ++r) {
    for (int64_t c = 0; c < i; ++c) {
      const double g = (double)bf16_to_f32(gu[r * 2 * i + c]);
      const double u = (double)bf16_to_f32(gu[r * 2 * i + i + c]);
      const double v = g / (1.0 + exp(-g)) * u;
      uint16_t near, alt;
      int a;
      bf16_neighbours(v, rel, &near, &alt, &a);
      h[r * i + c] = near;
      if (other) {
        other[r * i + c] = alt;
        amb[r * i + c] = (uint8_t)a;
      }
    }
  }
}

/* Codes of bf16 rows under given per-row scales: clamp(rne(fl32(a / s)), -127, 127), the
 * code step of the row quantizer with the scale fixed (q: [r, k]). */
void ref_codes_with_scale(const uint16_t* a, const float* s, int64_t r, int64_t k, int8_t* q) {
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < r; ++row)
    for (int64_t j = 0; j < k; ++j) {
      float c = round_half_even(bf16_to_f32(a[row * k + j]) / s[row]);
      if (c > 127.0f) c = 127.0f;
      if (c < -127.0f) c = -127.0f;
      q[row * k + j] = (int8_t)c;
    }
}
