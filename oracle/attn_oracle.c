/*
 * Exact-attention oracle: O = softmax(scale * Q K^T + mask) V and its
 * natural-log log-sum-exp, evaluated row by row in IEEE double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the GPU path is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg load it; the product
 * library never links it, and it shares no code, header or table with the
 * GPU kernels.
 *
 * What is computed, and where the pages define it:
 *  - Operation and layout: ffpa-attn "API Reference" (readthedocs),
 *    ffpa_attn_func: Q is [B, Nh_q, Nq, D], K and V are [B, Nh_kv, Nkv, D],
 *    the output is [B, Nh_q, Nq, D] holding softmax(scale * Q K^T) V.
 *  - Scale: same page, parameter "scale": applied to Q K^T before the
 *    softmax; 1/sqrt(D) when not given (the caller passes the value).
 *  - Grouped heads: same page, parameter "key": Nh_q is a multiple of Nh_kv
 *    and group_size = Nh_q / Nh_kv.  Query head h reads KV head
 *    floor(h / group_size) (consecutive query heads share a KV head; this is
 *    the reading documented with the build, equal to repeating every KV head
 *    group_size times).
 *  - Causal: same page, parameter "is_causal": query row r attends to key k
 *    only when k <= r + (Nkv - Nq) (queries aligned to the tail of the keys).
 *  - Mask: same page, parameter "attn_mask": broadcastable to
 *    [B, Nh_q, Nq, Nkv]; a boolean entry that is true takes part, a false one
 *    is excluded; a floating entry is an additive bias.  The bias is added
 *    after scaling, i.e. the logit is scale * q.k + bias.
 *  - LSE: the same page's varlen entry returns an fp32 log-sum-exp per query
 *    row; here it is the natural log of sum_k exp(logit_k) over the row.
 *
 * A row whose logits are all -inf (every key masked) has no defined softmax;
 * by the convention documented with the build its output row is 0 and its
 * LSE is -inf.
 *
 * Inputs are the raw 16-bit patterns of bf16 or fp16 values, or the bytes of
 * fp8 e4m3 values (the FP8 attention of the ffpa-attn README, "Latest News"
 * and "End-to-End Inference"), all of which widen to double exactly.  fp8
 * inputs come with per-head dequantisation factors (the "scale folding" the
 * skill descriptions on the skillsmp page name): the value a byte stands
 * for is descale[b, head] times its e4m3 value, and the attention above is
 * taken over those values.  Built without fast-math so IEEE infinities
 * behave.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_FP16 = 1, OR_E4M3 = 2 };
enum { OR_MASK_NONE = 0, OR_MASK_BOOL_U8 = 1, OR_MASK_ADD_F32 = 2, OR_MASK_ADD_BF16 = 3, OR_MASK_ADD_FP16 = 4 };

/* Planted-mistake switches, used only by the tests that show the oracle's
 * pins can tell a wrong oracle from a right one.  0 is the real oracle. */
enum {
  OR_FAULT_NONE = 0,
  OR_FAULT_TOPLEFT_CAUSAL = 1, /* k <= r instead of k <= r + Nkv - Nq */
  OR_FAULT_HEAD_MODULO = 2,    /* KV head h % Hkv instead of h / group */
  OR_FAULT_MASK_BEFORE_SCALE = 3, /* scale * (q.k + bias) */
  OR_FAULT_LSE_LOG2 = 4,       /* LSE reported in base 2 */
  OR_FAULT_DROP_LAST_KEY = 5,  /* sums stop one key early */
  OR_FAULT_V_TRANSPOSED = 6    /* reads V[d][k] instead of V[k][d] */
};

/* bf16 is the upper half of an IEEE binary32. */
static double widen_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double widen_fp16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexp((double)(f | 0x400), e - 25); /* (1 + f/1024) * 2^(e-15) */
  return sign ? -mag : mag;
}

/* OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits;
 * no infinities; exponent 15 with fraction 7 is NaN; exponent 0 holds the subnormals f * 2^-9. */
static double widen_e4m3(uint8_t x) {
  int sign = (x >> 7) & 1;
  int e = (x >> 3) & 0xf;
  int f = x & 0x7;
  double mag;
  if (e == 0)
    mag = ldexp((double)f, -9); /* f/8 * 2^(1-7) */
  else if (e == 15 && f == 7)
    mag = NAN;
  else
    mag = ldexp((double)(f | 0x8), e - 10); /* (1 + f/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

double oracle_e4m3_value(uint8_t x) { return widen_e4m3(x); }

/* Element i of a tensor of the given format, widened exactly. */
static double elem(const void* base, int64_t i, int dtype) {
  switch (dtype) {
    case OR_FP16: return widen_fp16(((const uint16_t*)base)[i]);
    case OR_E4M3: return widen_e4m3(((const uint8_t*)base)[i]);
    default: return widen_bf16(((const uint16_t*)base)[i]);
  }
}

/* The bias mu(b,h,r,k) of the mask, or 0 / -inf for a boolean mask. */
static double mask_term(const void* mask, int kind, int64_t off) {
  switch (kind) {
    case OR_MASK_BOOL_U8: return ((const uint8_t*)mask)[off] ? 0.0 : -INFINITY;
    case OR_MASK_ADD_F32: return (double)((const float*)mask)[off];
    case OR_MASK_ADD_BF16: return widen_bf16(((const uint16_t*)mask)[off]);
    case OR_MASK_ADD_FP16: return widen_fp16(((const uint16_t*)mask)[off]);
    default: return 0.0;
  }
}

/* Planted mistakes of the fp8 dequantisation (tests of its pins only). */
enum {
  OR_FAULT_Q8_KSCALE_QHEAD = 101, /* K's factor taken at the query head's index, not its KV head's */
  OR_FAULT_Q8_NO_VSCALE = 102,    /* V's factor left out */
  OR_FAULT_Q8_DIVIDE = 103        /* the factors divide instead of multiply */
};

/* The per-head factor of tensor t for (b, head); NULL means 1. */
static double factor(const float* f, int64_t b, int64_t heads, int64_t head, int fault) {
  if (f == NULL) return 1.0;
  const double x = (double)f[b * heads + head];
  return fault == OR_FAULT_Q8_DIVIDE ? 1.0 / x : x;
}

static int attn_rows(const void* q, const void* k, const void* v, const float* q_f, const float* k_f,
                     const float* v_f, const void* mask, int mask_kind, int64_t msb, int64_t msh, int64_t msq,
                     int64_t msk, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                     double scale, int is_causal, int dtype, const int64_t* rows, int64_t nrows, double* O_out,
                     double* LSE_out, double* P_out, int nthreads, int fault);

/*
 * Computes the rows listed in `rows` (flat indices (b*Hq + h)*Nq + r).
 * O_out is nrows x D, LSE_out is nrows, P_out (optional) is nrows x Nkv and
 * receives the softmax probabilities exp(logit - LSE).
 * Mask strides are in elements; a zero stride broadcasts that dimension.
 * Returns 0 on success, -1 on bad arguments, -2 if memory runs out.
 */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, const void* mask, int mask_kind,
                     int64_t msb, int64_t msh, int64_t msq, int64_t msk, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nkv, int64_t D, double scale, int is_causal, int dtype,
                     const int64_t* rows, int64_t nrows, double* O_out, double* LSE_out, double* P_out,
                     int nthreads, int fault) {
  if (dtype != OR_BF16 && dtype != OR_FP16) return -1;
  return attn_rows(q, k, v, NULL, NULL, NULL, mask, mask_kind, msb, msh, msq, msk, B, Hq, Hkv, Nq, Nkv, D, scale,
                   is_causal, dtype, rows, nrows, O_out, LSE_out, P_out, nthreads, fault);
}

/* The same rows for fp8 e4m3 inputs (bytes) with per-head factors q_f [B, Hq], k_f and v_f [B, Hkv]
 * (NULL: 1): the attention of the tensors whose elements are factor * e4m3 value. */
int oracle_attn_rows_e4m3(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_f,
                          const float* k_f, const float* v_f, const void* mask, int mask_kind, int64_t msb,
                          int64_t msh, int64_t msq, int64_t msk, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                          int64_t Nkv, int64_t D, double scale, int is_causal, const int64_t* rows, int64_t nrows,
                          double* O_out, double* LSE_out, double* P_out, int nthreads, int fault) {
  return attn_rows(q, k, v, q_f, k_f, v_f, mask, mask_kind, msb, msh, msq, msk, B, Hq, Hkv, Nq, Nkv, D, scale,
                   is_causal, OR_E4M3, rows, nrows, O_out, LSE_out, P_out, nthreads, fault);
}

static int attn_rows(const void* q, const void* k, const void* v, const float* q_f, const float* k_f,
                     const float* v_f, const void* mask, int mask_kind, int64_t msb, int64_t msh, int64_t msq,
                     int64_t msk, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D,
                     double scale, int is_causal, int dtype, const int64_t* rows, int64_t nrows, double* O_out,
                     double* LSE_out, double* P_out, int nthreads, int fault) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1 || Hq % Hkv != 0) return -1;
  if (mask_kind != OR_MASK_NONE && mask == NULL) return -1;
  const int64_t group = Hq / Hkv;
  const int64_t shift = Nkv - Nq; /* tail alignment of the causal mask */
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Nkv);
    double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
    if (!s || !qrow) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t i = 0; i < nrows; ++i) {
      if (failed) continue;
      const int64_t idx = rows[i];
      const int64_t r = idx % Nq;
      const int64_t h = (idx / Nq) % Hq;
      const int64_t b = idx / (Nq * Hq);
      const int64_t hk = fault == OR_FAULT_HEAD_MODULO ? h % Hkv : h / group;
      const int64_t qp = ((b * Hq + h) * Nq + r) * D; /* element offsets of the row and of the KV head */
      const int64_t kp = (b * Hkv + hk) * Nkv * D;
      const int64_t vp = kp;
      /* per-head dequantisation factors (1 for 16-bit inputs, whose elements are used as they are) */
      const double fq = factor(q_f, b, Hq, h, fault);
      const double fk = fault == OR_FAULT_Q8_KSCALE_QHEAD ? factor(k_f, b, Hq, h, fault) : factor(k_f, b, Hkv, hk, fault);
      const double fv = fault == OR_FAULT_Q8_NO_VSCALE ? 1.0 : factor(v_f, b, Hkv, hk, fault);
      for (int64_t d = 0; d < D; ++d) qrow[d] = elem(q, qp + d, dtype) * fq;
      int64_t nk = fault == OR_FAULT_DROP_LAST_KEY && Nkv > 1 ? Nkv - 1 : Nkv;
      const int64_t last_visible = fault == OR_FAULT_TOPLEFT_CAUSAL ? r : r + shift;

      /* logits and their maximum */
      double m = -INFINITY;
      for (int64_t kk = 0; kk < Nkv; ++kk) {
        double logit;
        if (kk >= nk || (is_causal && kk > last_visible)) {
          logit = -INFINITY;
        } else {
          double dot = 0.0;
          const int64_t krow = kp + kk * D;
          for (int64_t d = 0; d < D; ++d) dot += qrow[d] * (elem(k, krow + d, dtype) * fk);
          double mu = mask_kind ? mask_term(mask, mask_kind, b * msb + h * msh + r * msq + kk * msk) : 0.0;
          logit = fault == OR_FAULT_MASK_BEFORE_SCALE ? scale * (dot + mu) : scale * dot + mu;
        }
        s[kk] = logit;
        if (logit > m) m = logit;
      }

      double* orow = O_out + i * D;
      if (m == -INFINITY) { /* every key excluded */
        LSE_out[i] = -INFINITY;
        for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
        if (P_out)
          for (int64_t kk = 0; kk < Nkv; ++kk) P_out[i * Nkv + kk] = 0.0;
        continue;
      }
      double sum = 0.0;
      for (int64_t kk = 0; kk < Nkv; ++kk) sum += exp(s[kk] - m);
      const double lse = m + log(sum);
      LSE_out[i] = fault == OR_FAULT_LSE_LOG2 ? lse / log(2.0) : lse;

      for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
      for (int64_t kk = 0; kk < Nkv; ++kk) {
        const double p = exp(s[kk] - lse);
        if (P_out) P_out[i * Nkv + kk] = p;
        if (p == 0.0) continue;
        if (fault == OR_FAULT_V_TRANSPOSED) {
          /* reads V as if it were stored [D][Nkv] (only meaningful when D == Nkv) */
          for (int64_t d = 0; d < D; ++d) orow[d] += p * (elem(v, vp + (d % Nkv) * D + (kk % D), dtype) * fv);
        } else {
          const int64_t vrow = vp + kk * D;
          for (int64_t d = 0; d < D; ++d) orow[d] += p * (elem(v, vrow + d, dtype) * fv);
        }
      }
    }
    free(s);
    free(qrow);
  }
  return failed ? -2 : 0;
}

/* Number of keys row r may see under the tail-aligned causal rule. */
int64_t oracle_causal_visible(int64_t r, int64_t Nq, int64_t Nkv) {
  int64_t last = r + (Nkv - Nq);
  if (last < 0) return 0;
  return last + 1 < Nkv ? last + 1 : Nkv;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
