/*
 * Memory and undefined-behaviour check of the oracle (test infrastructure,
 * like the rest of oracle/): tests/test_oracle_sanitized.py builds this file
 * together with attn_oracle.c under AddressSanitizer and UBSan and runs it.
 * It calls every exported function on small synthetic problems in every
 * storage type and masking mode (ragged lengths, an empty sequence, more
 * query rows than keys, no keys at all), with every buffer allocated at its
 * exact size, so a read or write past any of them is reported.  It checks no
 * arithmetic (the pins do that): the exit status is 0 when every call
 * returned its documented status and no output holds a NaN.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attn_fwd(const void* q, const void* k, const void* v, int dtype, double* o, double* lse, int B, int Hq,
                    int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens, int window, double scale,
                    int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo, int threads, int causal);
int oracle_attn_fwd_rows(const void* q, const void* k, const void* v, int dtype, double* o, double* lse, int B,
                         int Hq, int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens, int window,
                         double scale, const int64_t* rows, int64_t nrows, int threads, int causal);
int64_t oracle_attn_probs(const void* q, const void* k, int dtype, int B, int Hq, int Hkv, int Q, int K, int D,
                          const int32_t* seqlens, int window, double scale, int b, int h, int qi, double* p_out,
                          int causal);
int oracle_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype, double* dq, double* dk,
                    double* dv, int B, int Hq, int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens,
                    int window, double scale, int threads, int causal);
int oracle_attn_bwd_rows(const void* q, const void* k, const void* v, const void* dout, int dtype, const int64_t* rows,
                         int64_t nrows, double* dq_out, int B, int Hq, int Hkv, int Q, int K, int D, int Dv,
                         const int32_t* seqlens, int window, double scale, int threads, int causal);
int oracle_attn_bwd_keys(const void* q, const void* k, const void* v, const void* dout, int dtype, const int64_t* keys,
                         int64_t nkeys, double* dk_out, double* dv_out, int B, int Hq, int Hkv, int Q, int K, int D,
                         int Dv, const int32_t* seqlens, int window, double scale, int threads, int causal);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double next_unit(void) { /* xorshift64*, uniform in [-1, 1) */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}

/* n elements of storage type dtype (0 bf16, 1 fp32, 2 fp16, 3 fp64), exactly n * size bytes. */
static void* make_tensor(int dtype, int64_t n) {
  const size_t esz = dtype == 3 ? 8 : (dtype == 1 ? 4 : 2);
  unsigned char* p = (unsigned char*)malloc(n > 0 ? (size_t)n * esz : 1);
  for (int64_t i = 0; i < n; ++i) {
    const double x = 2.0 * next_unit();
    if (dtype == 3) {
      memcpy(p + 8 * i, &x, 8);
    } else if (dtype == 1) {
      const float f = (float)x;
      memcpy(p + 4 * i, &f, 4);
    } else if (dtype == 0) {
      const float f = (float)x;
      uint32_t u;
      memcpy(&u, &f, 4);
      const uint16_t h = (uint16_t)(u >> 16); /* truncation: any bf16 pattern will do */
      memcpy(p + 2 * i, &h, 2);
    } else {
      /* binary16 with exponent 12..16 (|x| in [1/8, 4)), random sign and mantissa */
      const uint16_t h = (uint16_t)((x < 0 ? 0x8000u : 0u) | ((12u + (uint32_t)(fabs(x) * 2.4)) << 10) |
                                    ((uint32_t)(fabs(next_unit()) * 1023.0)));
      memcpy(p + 2 * i, &h, 2);
    }
  }
  return p;
}

static int failures = 0;
static void expect(int cond, const char* what, int dtype, int causal, int window) {
  if (!cond) {
    fprintf(stderr, "FAIL %s (dtype %d causal %d window %d)\n", what, dtype, causal, window);
    ++failures;
  }
}
static int no_nan(const double* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (isnan(x[i])) return 0;
  return 1;
}

static void run_case(int dtype, int B, int Hq, int Hkv, int Q, int K, int D, int Dv, const int32_t* seq_host,
                     int window, int causal) {
  const double scale = 0.37;
  const int64_t nq = (int64_t)B * Hq * Q * D, nk = (int64_t)B * Hkv * K * D, nv = (int64_t)B * Hkv * K * Dv;
  const int64_t rows = (int64_t)B * Hq * Q, no = rows * Dv, keys = (int64_t)B * Hkv * K;
  void* q = make_tensor(dtype, nq);
  void* k = make_tensor(dtype, nk);
  void* v = make_tensor(dtype, nv);
  void* dout = make_tensor(dtype, no);
  int32_t* seq = NULL;
  if (seq_host) {
    seq = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
    memcpy(seq, seq_host, sizeof(int32_t) * (size_t)B);
  }
  double* o = (double*)malloc(sizeof(double) * (size_t)(no > 0 ? no : 1));
  double* lse = (double*)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1));
  expect(oracle_attn_fwd(q, k, v, dtype, o, lse, B, Hq, Hkv, Q, K, D, Dv, seq, window, scale, D, D, Dv, Dv, 2,
                         causal) == 0,
         "fwd status", dtype, causal, window);
  expect(no_nan(o, no) && no_nan(lse, rows), "fwd values", dtype, causal, window);

  /* every third row, in reverse order */
  const int64_t nsel = (rows + 2) / 3;
  int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nsel > 0 ? nsel : 1));
  for (int64_t i = 0; i < nsel; ++i) sel[i] = rows - 1 - 3 * i;
  double* ro = (double*)malloc(sizeof(double) * (size_t)(nsel * Dv > 0 ? nsel * Dv : 1));
  double* rl = (double*)malloc(sizeof(double) * (size_t)(nsel > 0 ? nsel : 1));
  expect(oracle_attn_fwd_rows(q, k, v, dtype, ro, rl, B, Hq, Hkv, Q, K, D, Dv, seq, window, scale, sel, nsel, 2,
                              causal) == 0,
         "rows status", dtype, causal, window);
  expect(no_nan(ro, nsel * Dv) && no_nan(rl, nsel), "rows values", dtype, causal, window);

  if (rows > 0) {
    double* pr = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    expect(oracle_attn_probs(q, k, dtype, B, Hq, Hkv, Q, K, D, seq, window, scale, B - 1, Hq - 1, Q - 1, pr,
                             causal) >= 0,
           "probs status", dtype, causal, window);
    expect(no_nan(pr, K), "probs values", dtype, causal, window);
    free(pr);
  }

  double* dq = (double*)malloc(sizeof(double) * (size_t)(nq > 0 ? nq : 1));
  double* dk = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
  double* dv = (double*)malloc(sizeof(double) * (size_t)(nv > 0 ? nv : 1));
  expect(oracle_attn_bwd(q, k, v, dout, dtype, dq, dk, dv, B, Hq, Hkv, Q, K, D, Dv, seq, window, scale, 2,
                         causal) == 0,
         "bwd status", dtype, causal, window);
  expect(no_nan(dq, nq) && no_nan(dk, nk) && no_nan(dv, nv), "bwd values", dtype, causal, window);
  double* sdq = (double*)malloc(sizeof(double) * (size_t)(nsel * D > 0 ? nsel * D : 1));
  expect(oracle_attn_bwd_rows(q, k, v, dout, dtype, sel, nsel, sdq, B, Hq, Hkv, Q, K, D, Dv, seq, window, scale, 2,
                              causal) == 0,
         "bwd rows status", dtype, causal, window);
  expect(no_nan(sdq, nsel * D), "bwd rows values", dtype, causal, window);
  const int64_t nkey = (keys + 1) / 2;
  int64_t* ksel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nkey > 0 ? nkey : 1));
  for (int64_t i = 0; i < nkey; ++i) ksel[i] = 2 * i;
  double* sdk = (double*)malloc(sizeof(double) * (size_t)(nkey * D > 0 ? nkey * D : 1));
  double* sdv = (double*)malloc(sizeof(double) * (size_t)(nkey * Dv > 0 ? nkey * Dv : 1));
  expect(oracle_attn_bwd_keys(q, k, v, dout, dtype, ksel, nkey, sdk, sdv, B, Hq, Hkv, Q, K, D, Dv, seq, window,
                              scale, 2, causal) == 0,
         "bwd keys status", dtype, causal, window);
  expect(no_nan(sdk, nkey * D) && no_nan(sdv, nkey * Dv), "bwd keys values", dtype, causal, window);

  /* Argument errors are reported, not acted on. */
  if (seq && B > 0) {
    const int32_t saved = seq[0];
    seq[0] = K + 1;
    expect(oracle_attn_fwd(q, k, v, dtype, o, lse, B, Hq, Hkv, Q, K, D, Dv, seq, window, scale, D, D, Dv, Dv, 2,
                           causal) == -2,
           "length past K refused", dtype, causal, window);
    seq[0] = saved;
  }
  int64_t bad_row = rows;
  expect(oracle_attn_fwd_rows(q, k, v, dtype, ro, rl, B, Hq, Hkv, Q, K, D, Dv, seq, window, scale, &bad_row, 1, 2,
                              causal) == -1,
         "row out of range refused", dtype, causal, window);

  free(q); free(k); free(v); free(dout); free(seq); free(o); free(lse); free(sel); free(ro); free(rl);
  free(dq); free(dk); free(dv); free(sdq); free(ksel); free(sdk); free(sdv);
}

int main(void) {
  const int32_t ragged[2] = {13, 0}, partial[2] = {7, 13}, short_keys[3] = {4, 1, 0};
  int n = 0;
  for (int dtype = 0; dtype <= 3; ++dtype) {
    for (int mode = 0; mode < 4; ++mode) {
      const int causal = mode != 3, window = mode == 1 ? 3 : (mode == 2 ? 1 : 0);
      run_case(dtype, 2, 4, 2, 5, 13, 8, 12, ragged, window, causal);
      run_case(dtype, 2, 4, 2, 5, 13, 16, 8, partial, window, causal);
      run_case(dtype, 2, 6, 3, 5, 13, 8, 8, NULL, window, causal);
      run_case(dtype, 3, 2, 1, 9, 4, 8, 8, short_keys, window, causal); /* more query rows than keys */
      run_case(dtype, 1, 2, 2, 3, 0, 8, 8, NULL, window, causal);       /* no keys at all */
      n += 5;
    }
  }
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("ok: %d cases\n", n);
  return 0;
}
