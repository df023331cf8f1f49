/* Drives the C oracle (attn_oracle.c) on small inputs of every kind it accepts - bf16 and fp16,
 * each mask kind with broadcast strides, causal, grouped heads, the probability output, the fp8
 * e4m3 form, one and two threads - and with invalid arguments.  Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer, so that an out-of-bounds access or undefined behaviour fails the run;
 * the values themselves are pinned elsewhere. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, const void* mask, int mask_kind,
                     int64_t msb, int64_t msh, int64_t msq, int64_t msk, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nkv, int64_t D, double scale, int is_causal, int dtype,
                     const int64_t* rows, int64_t nrows, double* O_out, double* LSE_out, double* P_out,
                     int nthreads, int fault);
int oracle_attn_rows_e4m3(const uint8_t* q, const uint8_t* k, const uint8_t* v, const float* q_f,
                          const float* k_f, const float* v_f, const void* mask, int mask_kind, int64_t msb,
                          int64_t msh, int64_t msq, int64_t msk, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                          int64_t Nkv, int64_t D, double scale, int is_causal, const int64_t* rows, int64_t nrows,
                          double* O_out, double* LSE_out, double* P_out, int nthreads, int fault);
double oracle_e4m3_value(uint8_t x);
int64_t oracle_causal_visible(int64_t r, int64_t Nq, int64_t Nkv);

static uint32_t lcg = 12345u;
static uint32_t next(void) { return lcg = lcg * 1664525u + 1013904223u; }
/* a bf16 / fp16 bit pattern of a value in about [-2, 2] */
static uint16_t rnd16(int fp16) {
  const float x = ((int)(next() >> 9) - (1 << 22)) / (float)(1 << 22) * 2.0f;
  union { float f; uint32_t u; } c = {x};
  if (!fp16) return (uint16_t)(c.u >> 16);
  /* fp16: sign, exponent rebased, 10 mantissa bits (|x| <= 2, no overflow) */
  const uint32_t s = (c.u >> 16) & 0x8000u;
  const int e = (int)((c.u >> 23) & 0xff) - 127 + 15;
  if (e <= 0) return (uint16_t)s;
  return (uint16_t)(s | ((uint32_t)e << 10) | ((c.u >> 13) & 0x3ffu));
}

int main(void) {
  int failures = 0;
  const int64_t B = 2, Hq = 4, Hkv = 2, Nq = 9, Nkv = 13, D = 24;
  const int64_t nq = B * Hq * Nq * D, nk = B * Hkv * Nkv * D;
  uint16_t* q = malloc(nq * 2);
  uint16_t* k = malloc(nk * 2);
  uint16_t* v = malloc(nk * 2);
  uint8_t *q8 = malloc(nq), *k8 = malloc(nk), *v8 = malloc(nk);
  float qf[8], kf[4], vf[4];
  float* mf = malloc(B * Nq * Nkv * 4);
  uint8_t* mb = malloc(Nq * Nkv);
  uint16_t* m16 = malloc(Hq * Nq * Nkv * 2);
  int64_t rows[B * Hq * Nq];
  double *O = malloc(B * Hq * Nq * D * 8), *L = malloc(B * Hq * Nq * 8), *Pp = malloc(B * Hq * Nq * Nkv * 8);
  for (int64_t r = 0; r < B * Hq * Nq; ++r) rows[r] = r;
  for (int dt = 0; dt < 2; ++dt) {
    for (int64_t i = 0; i < nq; ++i) q[i] = rnd16(dt);
    for (int64_t i = 0; i < nk; ++i) k[i] = rnd16(dt), v[i] = rnd16(dt);
    for (int64_t i = 0; i < B * Nq * Nkv; ++i) mf[i] = (next() % 7 == 0) ? -INFINITY : (float)(next() % 100) / 50.0f;
    for (int64_t i = 0; i < Nq * Nkv; ++i) mb[i] = (uint8_t)(next() % 3 != 0);
    for (int64_t i = 0; i < Hq * Nq * Nkv; ++i) m16[i] = rnd16(dt);
    for (int causal = 0; causal < 2; ++causal)
      for (int th = 1; th <= 2; ++th) {
        /* no mask; f32 [B,1,Nq,Nkv]; bool [Nq,Nkv]; 16-bit [1,Hq,Nq,Nkv] */
        failures += oracle_attn_rows(q, k, v, NULL, 0, 0, 0, 0, 0, B, Hq, Hkv, Nq, Nkv, D, NAN, causal, dt, rows,
                                     B * Hq * Nq, O, L, Pp, th, 0) != 0;
        failures += oracle_attn_rows(q, k, v, mf, 2, Nq * Nkv, 0, Nkv, 1, B, Hq, Hkv, Nq, Nkv, D, 0.3, causal, dt,
                                     rows, B * Hq * Nq, O, L, NULL, th, 0) != 0;
        failures += oracle_attn_rows(q, k, v, mb, 1, 0, 0, Nkv, 1, B, Hq, Hkv, Nq, Nkv, D, NAN, causal, dt, rows + 3,
                                     5, O, L, Pp, th, 0) != 0;
        failures += oracle_attn_rows(q, k, v, m16, dt ? 4 : 3, 0, Nq * Nkv, Nkv, 1, B, Hq, Hkv, Nq, Nkv, D, NAN, causal,
                                     dt, rows, B * Hq * Nq, O, L, NULL, th, 0) != 0;
      }
    for (int64_t i = 0; i < B * Hq * Nq * D; ++i)
      if (isnan(O[i])) ++failures;
  }
  /* fp8 e4m3 codes (0x7f and 0xff are NaN: avoided), per-head factors */
  for (int64_t i = 0; i < nq; ++i) q8[i] = (uint8_t)(next() % 0x7e);
  for (int64_t i = 0; i < nk; ++i) k8[i] = (uint8_t)(next() % 0x7e) | (uint8_t)(next() & 0x80), v8[i] = (uint8_t)(next() % 0x7e);
  for (int i = 0; i < 8; ++i) qf[i] = 0.01f * (i + 1);
  for (int i = 0; i < 4; ++i) kf[i] = 0.02f * (i + 1), vf[i] = 0.5f;
  for (int causal = 0; causal < 2; ++causal) {
    failures += oracle_attn_rows_e4m3(q8, k8, v8, qf, kf, vf, mf, 2, Nq * Nkv, 0, Nkv, 1, B, Hq, Hkv, Nq, Nkv, D, NAN,
                                      causal, rows, B * Hq * Nq, O, L, Pp, 2, 0) != 0;
    failures += oracle_attn_rows_e4m3(q8, k8, v8, NULL, NULL, NULL, NULL, 0, 0, 0, 0, 0, B, Hq, Hkv, Nq, Nkv, D, NAN,
                                      causal, rows, B * Hq * Nq, O, L, NULL, 1, 0) != 0;
  }
  for (int c = 0; c < 256; ++c) (void)oracle_e4m3_value((uint8_t)c);
  for (int64_t r = 0; r < Nq; ++r) failures += oracle_causal_visible(r, Nq, Nkv) != r + (Nkv - Nq) + 1;
  /* invalid arguments are refused */
  failures += oracle_attn_rows(q, k, v, NULL, 0, 0, 0, 0, 0, B, Hq, Hkv, Nq, Nkv, D, NAN, 0, 9, rows, 1, O, L, NULL, 1,
                               0) != -1;
  failures += oracle_attn_rows(q, k, v, NULL, 0, 0, 0, 0, 0, B, 3, Hkv, Nq, Nkv, D, NAN, 0, 0, rows, 1, O, L, NULL, 1,
                               0) != -1;
  printf("%d failures\n", failures);
  free(q); free(k); free(v); free(q8); free(k8); free(v8); free(mf); free(mb); free(m16); free(O); free(L); free(Pp);
  return failures == 0 ? 0 : 1;
}
