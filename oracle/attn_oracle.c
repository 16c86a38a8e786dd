/*
 * Attention-forward oracle: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU implementation in double precision of what the GPU path
 * computes.  Only the tests, the package smoke check and the bench's CPU
 * baseline may load it; the product library never links or calls it, and it
 * shares no code, header or table with the GPU kernels.
 *
 * What is computed (LuisaCompute "Attention execution mapping" review,
 * section 1, the attention fixture paragraph): bottom-right causal
 * grouped-query attention, or, with causal = 0, the same attention without
 * the causal limit: every key k < K_b is legal for every row (section 7 of
 * the review names non-causal masks as an extension that needs its own
 * semantics and an independent oracle; this is that semantics, written as
 * plainly as the causal one).  Query head h reads kv-head h / (Hq/Hkv) (integer
 * division, contiguous groups); key k is legal for query row q when
 * k <= q + K - Q.  Readings where the pages are silent (each listed in the
 * design notes):
 *   - per-sequence length K_b replaces K in that offset, p(q) = q + K_b - Q,
 *     and only keys k < K_b exist (Laya "Fast backends", "Numerics": int32
 *     lengths, unequal lengths, empty sequences);
 *   - a sliding window W > 0 keeps the W keys p-W < k <= p (diagonal included);
 *   - a row with no legal key gets O = 0 and LSE = -inf (finite padded rows);
 *   - LSE is the natural log of the sum of exp(scale * q.k) over legal keys.
 * The softmax is written out in full: scores, their maximum, the exponentials,
 * their sum, the normalised weights and the weighted sum of V rows.  There is
 * no blocking and no online rescaling.
 *
 * Inputs are read element by element from bf16 (dtype 0, widened exactly),
 * fp32 (dtype 1) or IEEE binary16 (dtype 2, decoded exactly from its sign,
 * 5-bit exponent and 10-bit fraction; the Laya "Fast backends" page,
 * "Numerics", rounds GPU inputs to bf16 or fp16) storage and every operation
 * is done in double.  A window needs the causal limit (it is measured back from the
 * diagonal); causal = 0 with a window is rejected.  Row strides
 * (ldq, ldk, ldv, ldo) are in elements, so tests can embed V and O in wider
 * rows and check that columns beyond Dv are never read or written.
 *
 * The backward (oracle_attn_bwd) gives the gradients of the scalar
 * sum(dO * O) with respect to q, k and v (no cotangent on the LSE output):
 * per row, the weights P over the legal keys as above; dV[k] += P[k] dO;
 * dP[k] = dO . V[k]; the softmax Jacobian applied to dP, dS[k] = P[k] (dP[k]
 * - sum_j P[j] dP[j]); dQ = scale sum_k dS[k] K[k]; dK[k] += scale dS[k] q.
 * A kv-head's dK and dV sum the contributions of all its query heads.  These
 * are the chain rule through scores, softmax and the weighted sum, written in
 * those steps; the FlyDSL post ("FMHA through AOTriton") describes the
 * separate dQ and dK/dV passes of the GPU backward, which compute the same
 * quantities.  Input dtype 3 (double) exists for finite-difference checks.
 *
 * ORACLE_MUTANT (compile-time, tests only) plants one known mistake so the
 * pin tests can show they would catch it; the default build defines none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* IEEE 754 binary16: value = (-1)^s * 2^(e-15) * (1 + f/1024) for 0 < e < 31,
 * (-1)^s * 2^-14 * (f/1024) for e = 0, +-inf / NaN for e = 31. */
static double half_to_double(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double mag;
#if ORACLE_MUTANT == 15 /* exponent bias off by one */
  const int bias = 16;
#else
  const int bias = 15;
#endif
  if (e == 0)
    mag = ldexp((double)f, -24);
  else if (e == 31)
    mag = f ? NAN : INFINITY;
  else
    mag = ldexp(1.0 + (double)f / 1024.0, e - bias);
  return s ? -mag : mag;
}

static double load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == 0) {
    uint16_t h = ((const uint16_t*)base)[i];
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
  }
  if (dtype == 2) return half_to_double(((const uint16_t*)base)[i]);
  if (dtype == 3) return ((const double*)base)[i];
  return (double)((const float*)base)[i];
}

/* The legality predicate of one (row, key) pair. */
static int legal(int64_t k, int64_t p, int64_t Kb, int window, int causal) {
#if ORACLE_MUTANT == 14 /* causal limit applied to non-causal rows too */
  causal = 1;
#endif
#if ORACLE_MUTANT == 3 /* causal diagonal off by one */
  if (causal && !(k <= p + 1)) return 0;
#else
  if (causal && !(k <= p)) return 0;
#endif
  if (!(k >= 0 && k < Kb)) return 0;
#if ORACLE_MUTANT == 5 /* window one key too wide */
  if (window > 0 && !(k >= p - window)) return 0;
#else
  if (window > 0 && !(k > p - window)) return 0;
#endif
  return 1;
}

/*
 * Scores of one row (b, h, q) over all K key slots: scores[k] = scale * q.k for
 * legal keys, is_legal[k] marks them.  Returns the number of legal keys.
 */
static int64_t row_scores(const void* q, const void* k, int dtype, int Hq, int Hkv, int Q, int K, int D,
                          const int32_t* seqlens, int window, int causal, double scale, int64_t ldq, int64_t ldk,
                          int b, int h, int qi, double* scores, unsigned char* is_legal) {
#if ORACLE_MUTANT == 2 /* wrong GQA map: modulo instead of integer division */
  int kh = h % Hkv;
#else
  int kh = h / (Hq / Hkv);
#endif
#if ORACLE_MUTANT == 10 /* per-sequence lengths ignored */
  int64_t Kb = K;
#else
  int64_t Kb = seqlens ? seqlens[b] : K;
#endif
#if ORACLE_MUTANT == 4 /* top-left instead of bottom-right alignment */
  int64_t p = qi;
#else
  int64_t p = (int64_t)qi + Kb - Q;
#endif
  const int64_t qrow = (((int64_t)b * Hq + h) * Q + qi) * ldq;
  const int64_t kbase = ((int64_t)b * Hkv + kh) * (int64_t)K;
  int64_t n_legal = 0;
  for (int64_t kk = 0; kk < K; ++kk) {
    is_legal[kk] = (unsigned char)legal(kk, p, Kb, window, causal);
    if (!is_legal[kk]) continue;
    ++n_legal;
    double dot = 0.0;
#if ORACLE_MUTANT == 11 /* last channel of the dot product dropped */
    for (int d = 0; d < D - 1; ++d)
#else
    for (int d = 0; d < D; ++d)
#endif
      dot += load_elem(q, dtype, qrow + d) * load_elem(k, dtype, (kbase + kk) * ldk + d);
#if ORACLE_MUTANT == 1 /* scale dropped */
    scores[kk] = dot;
#elif ORACLE_MUTANT == 12 /* sign error */
    scores[kk] = -scale * dot;
#else
    scores[kk] = scale * dot;
#endif
  }
  return n_legal;
}

/* One output row (b, h, q): writes o_row[0..Dv) and *lse_out. */
static void oracle_row(const void* q, const void* k, const void* v, int dtype, int Hq, int Hkv, int Q, int K,
                       int D, int Dv, const int32_t* seqlens, int window, int causal, double scale, int64_t ldq,
                       int64_t ldk, int64_t ldv, int b, int h, int qi, double* o_row, double* lse_out,
                       double* scores, unsigned char* is_legal) {
  int64_t n_legal = row_scores(q, k, dtype, Hq, Hkv, Q, K, D, seqlens, window, causal, scale, ldq, ldk, b, h, qi,
                               scores, is_legal);
  if (n_legal == 0) {
    for (int j = 0; j < Dv; ++j) o_row[j] = 0.0;
    *lse_out = -INFINITY;
    return;
  }
  const int kh = h / (Hq / Hkv);
  const int64_t kbase = ((int64_t)b * Hkv + kh) * (int64_t)K;
  double m = -INFINITY;
  for (int64_t kk = 0; kk < K; ++kk)
    if (is_legal[kk] && scores[kk] > m) m = scores[kk];
  double l = 0.0;
  for (int64_t kk = 0; kk < K; ++kk)
    if (is_legal[kk]) l += exp(scores[kk] - m);
  for (int j = 0; j < Dv; ++j) {
    double acc = 0.0;
    for (int64_t kk = 0; kk < K; ++kk) {
      if (!is_legal[kk]) continue;
#if ORACLE_MUTANT == 7 /* V indexed as if transposed: channel and key swapped */
      double vv = load_elem(v, dtype, (kbase + (j % K)) * ldv + (kk % Dv));
#else
      double vv = load_elem(v, dtype, (kbase + kk) * ldv + j);
#endif
#if ORACLE_MUTANT == 9 /* weights not normalised by the sum */
      acc += exp(scores[kk] - m) * vv;
#else
      acc += exp(scores[kk] - m) / l * vv;
#endif
    }
    o_row[j] = acc;
  }
#if ORACLE_MUTANT == 6 /* row max left out of the log-sum-exp */
  *lse_out = log(l);
#elif ORACLE_MUTANT == 13 /* base-2 log */
  *lse_out = (m + log(l)) / log(2.0);
#else
  *lse_out = m + log(l);
#endif
}

static int check_args(int B, int Hq, int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens, int window,
                      int causal, int dtype) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Q < 0 || K < 0 || D < 0 || Dv < 0) return -1;
  if (dtype < 0 || dtype > 3) return -1;
  if (!causal && window > 0) return -1;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv != 0)) return -1;
  if (seqlens)
    for (int b = 0; b < B; ++b)
      if (seqlens[b] < 0 || seqlens[b] > K) return -2;
  return 0;
}

/*
 * Full problem: o[((b*Hq+h)*Q+q)*ldo + j], lse[(b*Hq+h)*Q+q].
 * Returns 0, -1 for bad sizes, -2 for a length outside [0, K], -3 on OOM.
 */
int oracle_attn_fwd(const void* q, const void* k, const void* v, int dtype, double* o, double* lse, int B, int Hq,
                    int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens, int window, double scale,
                    int64_t ldq, int64_t ldk, int64_t ldv, int64_t ldo, int threads, int causal) {
  int rc = check_args(B, Hq, Hkv, Q, K, D, Dv, seqlens, window, causal, dtype);
  if (rc) return rc;
  const int64_t rows = (int64_t)B * Hq * Q;
  int bad = 0;
#pragma omp parallel num_threads(threads > 0 ? threads : 1)
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    unsigned char* lg = (unsigned char*)malloc((size_t)(K > 0 ? K : 1));
    /* Every thread reaches the work-sharing loop; a thread without buffers only flags. */
#pragma omp for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
      if (!scores || !lg) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      int qi = (int)(r % Q);
      int h = (int)((r / Q) % Hq);
      int b = (int)(r / ((int64_t)Q * Hq));
      oracle_row(q, k, v, dtype, Hq, Hkv, Q, K, D, Dv, seqlens, window, causal, scale, ldq, ldk, ldv, b, h, qi,
                 o + r * ldo, lse + r, scores, lg);
    }
    free(scores);
    free(lg);
  }
  return bad ? -3 : 0;
}

/*
 * Selected rows only: rows[i] is the flat row index (b*Hq+h)*Q+q; the result
 * for rows[i] goes to o[i*Dv ...] and lse[i].  Used to check sampled outputs
 * of workloads too large to compute in full on the host.
 */
int oracle_attn_fwd_rows(const void* q, const void* k, const void* v, int dtype, double* o, double* lse, int B,
                         int Hq, int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens, int window,
                         double scale, const int64_t* rows, int64_t nrows, int threads, int causal) {
  int rc = check_args(B, Hq, Hkv, Q, K, D, Dv, seqlens, window, causal, dtype);
  if (rc) return rc;
  const int64_t total = (int64_t)B * Hq * Q;
  for (int64_t i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= total) return -1;
  int bad = 0;
#pragma omp parallel num_threads(threads > 0 ? threads : 1)
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    unsigned char* lg = (unsigned char*)malloc((size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
      if (!scores || !lg) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      int64_t r = rows[i];
      int qi = (int)(r % Q);
      int h = (int)((r / Q) % Hq);
      int b = (int)(r / ((int64_t)Q * Hq));
      oracle_row(q, k, v, dtype, Hq, Hkv, Q, K, D, Dv, seqlens, window, causal, scale, D, D, Dv, b, h, qi,
                 o + i * Dv, lse + i, scores, lg);
    }
    free(scores);
    free(lg);
  }
  return bad ? -3 : 0;
}

/*
 * The normalised weights P[k] of one row (0 for keys that are not legal),
 * so tests can check that they sum to one.  Returns the number of legal keys,
 * or a negative code as oracle_attn_fwd does.
 */
int64_t oracle_attn_probs(const void* q, const void* k, int dtype, int B, int Hq, int Hkv, int Q, int K, int D,
                          const int32_t* seqlens, int window, double scale, int b, int h, int qi, double* p_out,
                          int causal) {
  int rc = check_args(B, Hq, Hkv, Q, K, D, 1, seqlens, window, causal, dtype);
  if (rc) return rc;
  double* scores = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  unsigned char* lg = (unsigned char*)malloc((size_t)(K > 0 ? K : 1));
  if (!scores || !lg) {
    free(scores);
    free(lg);
    return -3;
  }
  int64_t n_legal =
      row_scores(q, k, dtype, Hq, Hkv, Q, K, D, seqlens, window, causal, scale, D, D, b, h, qi, scores, lg);
  double m = -INFINITY;
  for (int64_t kk = 0; kk < K; ++kk)
    if (lg[kk] && scores[kk] > m) m = scores[kk];
  double l = 0.0;
  for (int64_t kk = 0; kk < K; ++kk)
    if (lg[kk]) l += exp(scores[kk] - m);
  for (int64_t kk = 0; kk < K; ++kk) {
    p_out[kk] = 0.0;
    if (!lg[kk]) continue;
#if ORACLE_MUTANT == 9
    p_out[kk] = exp(scores[kk] - m);
#else
    p_out[kk] = exp(scores[kk] - m) / l;
#endif
  }
  free(scores);
  free(lg);
  return n_legal;
}

/*
 * Backward of one (batch, kv-head) group: every row of its query heads.
 * Adds into dk, dv of the group (zeroed by the caller) and writes dq rows.
 */
static void oracle_bwd_group(const void* q, const void* k, const void* v, const void* dout, int dtype, double* dq,
                             double* dk, double* dv, int Hq, int Hkv, int Q, int K, int D, int Dv,
                             const int32_t* seqlens, int window, int causal, double scale, int b, int kh,
                             double* scores, unsigned char* is_legal, double* pw, double* dp) {
  const int g = Hq / Hkv;
  const int64_t kbase = ((int64_t)b * Hkv + kh) * (int64_t)K;
  for (int hh = 0; hh < g; ++hh) {
    const int h = kh * g + hh;
    for (int qi = 0; qi < Q; ++qi) {
      const int64_t r = ((int64_t)b * Hq + h) * Q + qi;
      for (int d = 0; d < D; ++d) dq[r * D + d] = 0.0;
      int64_t n_legal = row_scores(q, k, dtype, Hq, Hkv, Q, K, D, seqlens, window, causal, scale, D, D, b, h, qi,
                                   scores, is_legal);
      if (n_legal == 0) continue;
      /* The row's weights, as in the forward. */
      double m = -INFINITY;
      for (int64_t kk = 0; kk < K; ++kk)
        if (is_legal[kk] && scores[kk] > m) m = scores[kk];
      double l = 0.0;
      for (int64_t kk = 0; kk < K; ++kk)
        if (is_legal[kk]) l += exp(scores[kk] - m);
      for (int64_t kk = 0; kk < K; ++kk) {
#if ORACLE_MUTANT == 18 /* dV from unnormalised weights */
        pw[kk] = is_legal[kk] ? exp(scores[kk] - m) : 0.0;
#else
        pw[kk] = is_legal[kk] ? exp(scores[kk] - m) / l : 0.0;
#endif
      }
      /* dV[k] += P[k] dO; dP[k] = dO . V[k]. */
      double delta = 0.0;
      for (int64_t kk = 0; kk < K; ++kk) {
        if (!is_legal[kk]) continue;
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j) {
          const double g_o = load_elem(dout, dtype, r * Dv + j);
#if ORACLE_MUTANT == 19 /* dV accumulated into the wrong kv-head's rows */
          const int64_t vrow = (((int64_t)b * Hkv + (h % Hkv)) * (int64_t)K + kk) * Dv;
#else
          const int64_t vrow = (kbase + kk) * Dv;
#endif
          dv[vrow + j] += pw[kk] * g_o;
          acc += g_o * load_elem(v, dtype, (kbase + kk) * Dv + j);
        }
        dp[kk] = acc;
        delta += pw[kk] * acc;
      }
      /* dS[k] = P[k] (dP[k] - delta); dQ += scale dS[k] K[k]; dK[k] += scale dS[k] q. */
      const int64_t qrow = r * D;
      for (int64_t kk = 0; kk < K; ++kk) {
        if (!is_legal[kk]) continue;
#if ORACLE_MUTANT == 16 /* the softmax Jacobian's delta term dropped */
        const double ds = pw[kk] * dp[kk];
#else
        const double ds = pw[kk] * (dp[kk] - delta);
#endif
        for (int d = 0; d < D; ++d) {
          dq[qrow + d] += scale * ds * load_elem(k, dtype, (kbase + kk) * D + d);
#if ORACLE_MUTANT == 17 /* scale missing from dK */
          dk[(kbase + kk) * D + d] += ds * load_elem(q, dtype, qrow + d);
#else
          dk[(kbase + kk) * D + d] += scale * ds * load_elem(q, dtype, qrow + d);
#endif
        }
      }
    }
  }
}

/*
 * Full backward: dq [B,Hq,Q,D], dk [B,Hkv,K,D], dv [B,Hkv,K,Dv] (dense rows),
 * dout [B,Hq,Q,Dv] in the input dtype.  Keys past K_b get zero gradients.
 * Returns 0, or a negative code as oracle_attn_fwd does.
 */
int oracle_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype, double* dq, double* dk,
                    double* dv, int B, int Hq, int Hkv, int Q, int K, int D, int Dv, const int32_t* seqlens,
                    int window, double scale, int threads, int causal) {
  int rc = check_args(B, Hq, Hkv, Q, K, D, Dv, seqlens, window, causal, dtype);
  if (rc) return rc;
  const int64_t groups = (int64_t)B * Hkv;
  memset(dk, 0, sizeof(double) * (size_t)(groups * K * D));
  memset(dv, 0, sizeof(double) * (size_t)(groups * K * Dv));
  if (Hq == 0 || Q == 0) return 0;
  int bad = 0;
#pragma omp parallel num_threads(threads > 0 ? threads : 1)
  {
    const size_t n = (size_t)(K > 0 ? K : 1);
    double* scores = (double*)malloc(sizeof(double) * n);
    unsigned char* lg = (unsigned char*)malloc(n);
    double* pw = (double*)malloc(sizeof(double) * n);
    double* dp = (double*)malloc(sizeof(double) * n);
#pragma omp for schedule(dynamic, 1)
    for (int64_t gi = 0; gi < groups; ++gi) {
      if (!scores || !lg || !pw || !dp) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      oracle_bwd_group(q, k, v, dout, dtype, dq, dk, dv, Hq, Hkv, Q, K, D, Dv, seqlens, window, causal, scale,
                       (int)(gi / Hkv), (int)(gi % Hkv), scores, lg, pw, dp);
    }
    free(scores);
    free(lg);
    free(pw);
    free(dp);
  }
  return bad ? -3 : 0;
}

/*
 * Backward on samples, for problems too large to differentiate in full on
 * the host.  The same steps as oracle_attn_bwd, restricted:
 *   oracle_attn_bwd_rows: dq of the listed flat rows (b*Hq+h)*Q+q, each from
 *     its own row (weights, dP, delta, dS), into dq_out[i*D ...];
 *   oracle_attn_bwd_keys: dk, dv of the listed flat keys (b*Hkv+kh)*K+k: every
 *     row of the kv-head's query heads contributes through its full weights,
 *     into dk_out[i*D ...] and dv_out[i*Dv ...].
 * Returns 0 or a negative code as oracle_attn_fwd does.
 */
int oracle_attn_bwd_rows(const void* q, const void* k, const void* v, const void* dout, int dtype, const int64_t* rows,
                         int64_t nrows, double* dq_out, int B, int Hq, int Hkv, int Q, int K, int D, int Dv,
                         const int32_t* seqlens, int window, double scale, int threads, int causal) {
  int rc = check_args(B, Hq, Hkv, Q, K, D, Dv, seqlens, window, causal, dtype);
  if (rc) return rc;
  const int64_t total = (int64_t)B * Hq * Q;
  for (int64_t i = 0; i < nrows; ++i)
    if (rows[i] < 0 || rows[i] >= total) return -1;
  int bad = 0;
#pragma omp parallel num_threads(threads > 0 ? threads : 1)
  {
    const size_t n = (size_t)(K > 0 ? K : 1);
    double* scores = (double*)malloc(sizeof(double) * n);
    unsigned char* lg = (unsigned char*)malloc(n);
    double* pw = (double*)malloc(sizeof(double) * n);
    double* dp = (double*)malloc(sizeof(double) * n);
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrows; ++i) {
      if (!scores || !lg || !pw || !dp) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      const int64_t r = rows[i];
      const int qi = (int)(r % Q), h = (int)((r / Q) % Hq), b = (int)(r / ((int64_t)Q * Hq));
      const int kh = h / (Hq / Hkv);
      const int64_t kbase = ((int64_t)b * Hkv + kh) * (int64_t)K;
      double* dq = dq_out + i * D;
      for (int d = 0; d < D; ++d) dq[d] = 0.0;
      if (row_scores(q, k, dtype, Hq, Hkv, Q, K, D, seqlens, window, causal, scale, D, D, b, h, qi, scores, lg) == 0)
        continue;
      double m = -INFINITY, l = 0.0, delta = 0.0;
      for (int64_t kk = 0; kk < K; ++kk)
        if (lg[kk] && scores[kk] > m) m = scores[kk];
      for (int64_t kk = 0; kk < K; ++kk)
        if (lg[kk]) l += exp(scores[kk] - m);
      for (int64_t kk = 0; kk < K; ++kk) {
        if (!lg[kk]) continue;
        pw[kk] = exp(scores[kk] - m) / l;
        double acc = 0.0;
        for (int j = 0; j < Dv; ++j)
          acc += load_elem(dout, dtype, r * Dv + j) * load_elem(v, dtype, (kbase + kk) * Dv + j);
        dp[kk] = acc;
        delta += pw[kk] * acc;
      }
      for (int64_t kk = 0; kk < K; ++kk) {
        if (!lg[kk]) continue;
        const double ds = pw[kk] * (dp[kk] - delta);
        for (int d = 0; d < D; ++d) dq[d] += scale * ds * load_elem(k, dtype, (kbase + kk) * D + d);
      }
    }
    free(scores);
    free(lg);
    free(pw);
    free(dp);
  }
  return bad ? -3 : 0;
}

int oracle_attn_bwd_keys(const void* q, const void* k, const void* v, const void* dout, int dtype, const int64_t* keys,
                         int64_t nkeys, double* dk_out, double* dv_out, int B, int Hq, int Hkv, int Q, int K, int D,
                         int Dv, const int32_t* seqlens, int window, double scale, int threads, int causal) {
  int rc = check_args(B, Hq, Hkv, Q, K, D, Dv, seqlens, window, causal, dtype);
  if (rc) return rc;
  const int64_t total = (int64_t)B * Hkv * K;
  for (int64_t i = 0; i < nkeys; ++i)
    if (keys[i] < 0 || keys[i] >= total) return -1;
  memset(dk_out, 0, sizeof(double) * (size_t)(nkeys * D));
  memset(dv_out, 0, sizeof(double) * (size_t)(nkeys * Dv));
  if (Hq == 0 || Q == 0) return 0;
  const int g = Hq / Hkv;
  int bad = 0;
  /* One pass over the rows of each (b, kv-head) group that holds a listed key. */
  for (int64_t gi = 0; gi < (int64_t)B * Hkv; ++gi) {
    int any = 0;
    for (int64_t i = 0; i < nkeys; ++i) any |= (keys[i] / K == gi);
    if (!any) continue;
    const int b = (int)(gi / Hkv), kh = (int)(gi % Hkv);
    const int64_t kbase = gi * (int64_t)K;
    const int64_t nrow = (int64_t)g * Q;
#pragma omp parallel num_threads(threads > 0 ? threads : 1)
    {
      const size_t n = (size_t)(K > 0 ? K : 1);
      double* scores = (double*)malloc(sizeof(double) * n);
      unsigned char* lg = (unsigned char*)malloc(n);
      double* pw = (double*)malloc(sizeof(double) * n);
      double* dp = (double*)malloc(sizeof(double) * n);
      double* tk = (double*)calloc((size_t)(nkeys * D + 1), sizeof(double));
      double* tv = (double*)calloc((size_t)(nkeys * Dv + 1), sizeof(double));
#pragma omp for schedule(dynamic, 4)
      for (int64_t ri = 0; ri < nrow; ++ri) {
        if (!scores || !lg || !pw || !dp || !tk || !tv) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        const int h = kh * g + (int)(ri / Q), qi = (int)(ri % Q);
        const int64_t r = ((int64_t)b * Hq + h) * Q + qi;
        if (row_scores(q, k, dtype, Hq, Hkv, Q, K, D, seqlens, window, causal, scale, D, D, b, h, qi, scores, lg) ==
            0)
          continue;
        double m = -INFINITY, l = 0.0, delta = 0.0;
        for (int64_t kk = 0; kk < K; ++kk)
          if (lg[kk] && scores[kk] > m) m = scores[kk];
        for (int64_t kk = 0; kk < K; ++kk)
          if (lg[kk]) l += exp(scores[kk] - m);
        for (int64_t kk = 0; kk < K; ++kk) {
          if (!lg[kk]) continue;
          pw[kk] = exp(scores[kk] - m) / l;
          double acc = 0.0;
          for (int j = 0; j < Dv; ++j)
            acc += load_elem(dout, dtype, r * Dv + j) * load_elem(v, dtype, (kbase + kk) * Dv + j);
          dp[kk] = acc;
          delta += pw[kk] * acc;
        }
        for (int64_t i = 0; i < nkeys; ++i) {
          if (keys[i] / K != gi) continue;
          const int64_t kk = keys[i] % K;
          if (!lg[kk]) continue;
          const double ds = pw[kk] * (dp[kk] - delta);
          for (int j = 0; j < Dv; ++j) tv[i * Dv + j] += pw[kk] * load_elem(dout, dtype, r * Dv + j);
          for (int d = 0; d < D; ++d) tk[i * D + d] += scale * ds * load_elem(q, dtype, r * D + d);
        }
      }
#pragma omp critical
      {
        if (tk && tv) {
          for (int64_t i = 0; i < nkeys * D; ++i) dk_out[i] += tk[i];
          for (int64_t i = 0; i < nkeys * Dv; ++i) dv_out[i] += tv[i];
        }
      }
      free(scores);
      free(lg);
      free(pw);
      free(dp);
      free(tk);
      free(tv);
    }
  }
  return bad ? -3 : 0;
}
