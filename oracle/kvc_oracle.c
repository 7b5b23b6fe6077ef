/*
 * kvc_oracle.c -- plain, slow, double-precision CPU reference of one
 * autoregressive KV-cache append + causal GQA softmax attention step.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test-suite, the smoke check and
 * the CPU-baseline leg of the benchmark, never by the product library.
 *
 * Every step cites the passage it follows.  "Page 1" is "Autoregressive
 * KV-cache append and causal attention" (biotorch problem
 * kv_cache_attention_step); "page 2" is "Fixed-capacity KV cache"
 * (aiengineeringfromscratch, practice kv-cache-append); "page 5" is
 * KempnerForge pull request 542 (lower-right causal mask for cached
 * multi-token appends).
 *
 * Nothing here is blocked, fused or reordered: each attention row is the
 * definition written out -- scores, max, exponentials, sum, division,
 * weighted sum of values -- in double.
 */
#include "kvc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int64_t elem_bytes(int dtype) { return dtype == 0 ? 4 : 2; }

/* Widen element idx of a dtype-0 (binary32) or dtype-1 (bfloat16) array to
 * double.  bfloat16 is the top half of a binary32 word, so the widening is
 * exact in both cases. */
static double load_elem(const void *base, int64_t idx, int dtype) {
  if (dtype == 0) return (double)((const float *)base)[idx];
  uint32_t word = (uint32_t)((const uint16_t *)base)[idx] << 16;
  float f;
  memcpy(&f, &word, sizeof f);
  return (double)f;
}

static int check_dims(int64_t B, int64_t Hq, int64_t Hk, int64_t Q, int64_t M,
                      int64_t D, int64_t Dv, int dtype) {
  /* Page 1, Required behavior: B, Hq, Hk, D, Dv, M >= 1, Q >= 0 and Hq a
   * multiple of Hk. */
  if (B < 1 || Hq < 1 || Hk < 1 || D < 1 || Dv < 1 || M < 1 || Q < 0)
    return KVC_ORACLE_ESHAPE;
  if (Hq % Hk != 0) return KVC_ORACLE_ESHAPE;
  if (dtype != 0 && dtype != 1) return KVC_ORACLE_EDTYPE;
  return KVC_ORACLE_OK;
}

/* Page 1, Required behavior: scale must be positive, default 1/sqrt(D) with
 * D the query/key width (page 2, Task, divides by sqrt(d_k) as well). */
static int resolve_scale(int has_scale, double scale, int64_t D, double *out) {
  if (!has_scale) {
    *out = 1.0 / sqrt((double)D);
    return KVC_ORACLE_OK;
  }
  if (!(scale > 0.0) || !isfinite(scale)) return KVC_ORACLE_ESCALE;
  *out = scale;
  return KVC_ORACLE_OK;
}

/* Row preparation.  Page 1, Required behavior: append_mask[b,:] must be a
 * run of Trues followed by Falses, its count n satisfies length + n <= M,
 * and 0 <= length <= M.  Page 1 leaves broken rows outside the contract;
 * page 2 (Task) rejects an append that does not fit and leaves the cache as
 * it was.  Reading taken here: a broken row is rejected, treated as n = 0,
 * and reported in its status. */
static int32_t row_prepare(const uint8_t *mask_row, int64_t Q, int64_t len,
                           int64_t M, int64_t *n_out) {
  int64_t n = 0, t;
  *n_out = 0;
  if (len < 0 || len > M) return KVC_ORACLE_ROW_BAD_LENGTH;
  while (n < Q && mask_row[n] != 0) n++;
  for (t = n; t < Q; t++)
    if (mask_row[t] != 0) return KVC_ORACLE_ROW_NOT_PREFIX;
  if (len + n > M) return KVC_ORACLE_ROW_OVERFLOW;
  *n_out = n;
  return KVC_ORACLE_ROW_OK;
}

int kvc_oracle_append(int64_t B, int64_t Hq, int64_t Hk, int64_t Q, int64_t M,
                      int64_t D, int64_t Dv, int dtype, const void *new_key,
                      const void *new_value, const void *key_cache,
                      const void *value_cache, const int64_t *lengths,
                      const uint8_t *append_mask, void *key_cache_out,
                      void *value_cache_out, int64_t *lengths_out,
                      int64_t *n_out, int32_t *row_status) {
  int rc = check_dims(B, Hq, Hk, Q, M, D, Dv, dtype);
  if (rc != KVC_ORACLE_OK) return rc;
  if (!key_cache || !value_cache || !lengths || !key_cache_out ||
      !value_cache_out || !lengths_out)
    return KVC_ORACLE_ENULL;
  if (Q > 0 && (!new_key || !new_value || !append_mask)) return KVC_ORACLE_ENULL;

  const int64_t e = elem_bytes(dtype);
  const uint8_t *nk = (const uint8_t *)new_key;
  const uint8_t *nv = (const uint8_t *)new_value;
  uint8_t *ko = (uint8_t *)key_cache_out;
  uint8_t *vo = (uint8_t *)value_cache_out;

  /* Page 1, Required behavior: the entire cache is returned and every entry
   * that is not written keeps its exact bits, the unused tail included.  The
   * copy is a byte copy, never a float conversion. */
  memcpy(key_cache_out, key_cache, (size_t)(B * Hk * M * D * e));
  memcpy(value_cache_out, value_cache, (size_t)(B * Hk * M * Dv * e));

  for (int64_t b = 0; b < B; b++) {
    int64_t n = 0;
    int32_t status = row_prepare(append_mask + b * Q, Q, lengths[b], M, &n);
    if (row_status) row_status[b] = status;
    if (n_out) n_out[b] = n;
    /* Page 1, Required behavior: new_key/value row t goes to slot
     * length + t, only for the True (prefix) append slots. */
    for (int64_t h = 0; h < Hk; h++) {
      for (int64_t t = 0; t < n; t++) {
        int64_t slot = lengths[b] + t;
        memcpy(ko + (((b * Hk + h) * M + slot) * D) * e,
               nk + (((b * Hk + h) * Q + t) * D) * e, (size_t)(D * e));
        memcpy(vo + (((b * Hk + h) * M + slot) * Dv) * e,
               nv + (((b * Hk + h) * Q + t) * Dv) * e, (size_t)(Dv * e));
      }
    }
    /* Page 1, Required behavior: the updated length is length + n; a
     * rejected row keeps its length (page 2, Examples: after the failed
     * append the length is still 3). */
    lengths_out[b] = lengths[b] + n;
  }
  return KVC_ORACLE_OK;
}

int kvc_oracle_attend_row(int64_t B, int64_t Hq, int64_t Hk, int64_t Q,
                          int64_t M, int64_t D, int64_t Dv, int dtype,
                          int has_scale, double scale, const void *query,
                          const void *key_updated, const void *value_updated,
                          int64_t old_len, int64_t n, int64_t b, int64_t hq,
                          int64_t t, double *attention_row,
                          double *context_row) {
  int rc = check_dims(B, Hq, Hk, Q, M, D, Dv, dtype);
  if (rc != KVC_ORACLE_OK) return rc;
  double sc;
  rc = resolve_scale(has_scale, scale, D, &sc);
  if (rc != KVC_ORACLE_OK) return rc;
  if (b < 0 || b >= B || hq < 0 || hq >= Hq || t < 0 || t >= Q)
    return KVC_ORACLE_ESHAPE;

  for (int64_t j = 0; j < M; j++) attention_row[j] = 0.0;
  for (int64_t d = 0; d < Dv; d++) context_row[d] = 0.0;

  /* Page 1, Required behavior: a query row is valid when its append slot is
   * True (t < n); invalid rows return zero attention and context. */
  if (t >= n) return KVC_ORACLE_OK;
  if (old_len < 0 || old_len + n > M) return KVC_ORACLE_ESHAPE;

  /* Page 1, Required behavior: query head hq reads KV head
   * floor(hq / (Hq / Hk)). */
  const int64_t group = Hq / Hk;
  const int64_t h = hq / group;

  /* Page 1, Required behavior: the valid query t may use slots
   * j <= old_length + t and j < new_length.  That is the lower-right causal
   * alignment of page 5 (Summary): appended token t sees every cached key
   * and the new keys up to its own position. */
  const int64_t new_len = old_len + n;
  int64_t last = old_len + t;
  if (last > new_len - 1) last = new_len - 1;

  /* Page 1, Required behavior: scores(q, k) = scale * dot(q, k). */
  const int64_t qoff = ((b * Hq + hq) * Q + t) * D;
  for (int64_t j = 0; j <= last; j++) {
    const int64_t koff = ((b * Hk + h) * M + j) * D;
    double dot = 0.0;
    for (int64_t d = 0; d < D; d++)
      dot += load_elem(query, qoff + d, dtype) *
             load_elem(key_updated, koff + d, dtype);
    attention_row[j] = sc * dot;
  }

  /* Page 1, Required behavior, and page 2, Constraints (scores above 1000
   * must give finite output): softmax taken after subtracting the row max. */
  double mx = attention_row[0];
  for (int64_t j = 1; j <= last; j++)
    if (attention_row[j] > mx) mx = attention_row[j];
  double z = 0.0;
  for (int64_t j = 0; j <= last; j++) {
    attention_row[j] = exp(attention_row[j] - mx);
    z += attention_row[j];
  }
  for (int64_t j = 0; j <= last; j++) attention_row[j] = attention_row[j] / z;

  /* Page 1, Required behavior: context = attention x updated values. */
  for (int64_t j = 0; j <= last; j++) {
    const int64_t voff = ((b * Hk + h) * M + j) * Dv;
    for (int64_t d = 0; d < Dv; d++)
      context_row[d] += attention_row[j] * load_elem(value_updated, voff + d, dtype);
  }
  return KVC_ORACLE_OK;
}

int kvc_oracle_step(int64_t B, int64_t Hq, int64_t Hk, int64_t Q, int64_t M,
                    int64_t D, int64_t Dv, int dtype, int has_scale,
                    double scale, const void *query, const void *new_key,
                    const void *new_value, const void *key_cache,
                    const void *value_cache, const int64_t *lengths,
                    const uint8_t *append_mask, void *key_cache_out,
                    void *value_cache_out, int64_t *lengths_out,
                    double *attention, double *context, int32_t *row_status) {
  int rc = check_dims(B, Hq, Hk, Q, M, D, Dv, dtype);
  if (rc != KVC_ORACLE_OK) return rc;
  double sc;
  rc = resolve_scale(has_scale, scale, D, &sc);
  if (rc != KVC_ORACLE_OK) return rc;
  if (Q > 0 && (!query || !attention || !context)) return KVC_ORACLE_ENULL;

  int64_t *n = (int64_t *)malloc((size_t)B * sizeof(int64_t));
  if (!n) return KVC_ORACLE_ENULL;
  rc = kvc_oracle_append(B, Hq, Hk, Q, M, D, Dv, dtype, new_key, new_value,
                         key_cache, value_cache, lengths, append_mask,
                         key_cache_out, value_cache_out, lengths_out, n,
                         row_status);
  if (rc == KVC_ORACLE_OK) {
    /* Page 1, Required behavior: Q = 0 gives empty attention and context;
     * otherwise every (b, hq, t) row is computed over the updated cache. */
    for (int64_t b = 0; b < B && rc == KVC_ORACLE_OK; b++)
      for (int64_t hq = 0; hq < Hq && rc == KVC_ORACLE_OK; hq++)
        for (int64_t t = 0; t < Q && rc == KVC_ORACLE_OK; t++) {
          const int64_t row = (b * Hq + hq) * Q + t;
          rc = kvc_oracle_attend_row(B, Hq, Hk, Q, M, D, Dv, dtype, 1, sc,
                                     query, key_cache_out, value_cache_out,
                                     lengths[b], n[b], b, hq, t,
                                     attention + row * M, context + row * Dv);
        }
  }
  free(n);
  return rc;
}

/* Read-only re-attention ("ClikaRT::ops::attention_over_cache", function
 * description): the cache is never written; sequence b's S_b queries are
 * the last S_b positions of its L_b cached ones (the query position follows
 * from the total cached length), so query t attends the prefix
 * j <= L_b - S_b + t -- the same lower-right alignment as the step.  The
 * per-head sink is one more logit in the softmax denominator that carries
 * no value row.  Reading taken here: the sink is compared with the scaled
 * scores as it is (it is not multiplied by the scale). */
int kvc_oracle_reattend(int64_t B, int64_t Hq, int64_t Hk, int64_t Q,
                        int64_t M, int64_t D, int64_t Dv, int dtype,
                        int has_scale, double scale, int64_t Tq,
                        const void *q, const int64_t *cu_q, const void *key,
                        const void *value, const int64_t *seqlens_k,
                        const double *sink, double *out, int32_t *status) {
  int rc = check_dims(B, Hq, Hk, Q, M, D, Dv, dtype);
  if (rc != KVC_ORACLE_OK) return rc;
  double sc;
  rc = resolve_scale(has_scale, scale, D, &sc);
  if (rc != KVC_ORACLE_OK) return rc;
  if (!q || !cu_q || !key || !value || !seqlens_k || !out || !status || Tq < 0)
    return KVC_ORACLE_ENULL;
  const int64_t G = Hq / Hk;
  int64_t i, b, t, h, j, d;
  for (i = 0; i < Tq * Hq * Dv; i++) out[i] = 0.0;
  for (b = 0; b < B; b++) {
    const int64_t L = seqlens_k[b], S = cu_q[b + 1] - cu_q[b];
    if (L < 0 || L > M) {
      status[b] = KVC_ORACLE_ROW_BAD_LENGTH;
      continue;
    }
    if (S < 0 || S > Q || S > L || cu_q[b] < 0 || cu_q[b + 1] > Tq) {
      status[b] = KVC_ORACLE_ROW_BAD_QUERIES;
      continue;
    }
    status[b] = KVC_ORACLE_ROW_OK;
    for (t = 0; t < S; t++) {
      const int64_t qrow = cu_q[b] + t, pos = L - S + t;
      for (h = 0; h < Hq; h++) {
        const int64_t kh = h / G;
        double *s = (double *)malloc((size_t)(pos + 1) * sizeof(double));
        double m = -INFINITY, z = 0.0;
        for (j = 0; j <= pos; j++) {
          double acc = 0.0;
          for (d = 0; d < D; d++)
            acc += load_elem(q, (qrow * Hq + h) * D + d, dtype) *
                   load_elem(key, ((b * Hk + kh) * M + j) * D + d, dtype);
          s[j] = sc * acc;
          if (s[j] > m) m = s[j];
        }
        if (sink && sink[h] > m) m = sink[h];
        for (j = 0; j <= pos; j++) z += exp(s[j] - m);
        if (sink) z += exp(sink[h] - m);
        double *o = out + (qrow * Hq + h) * Dv;
        for (j = 0; j <= pos; j++) {
          const double p = exp(s[j] - m) / z;
          for (d = 0; d < Dv; d++)
            o[d] += p * load_elem(value, ((b * Hk + kh) * M + j) * Dv + d, dtype);
        }
        free(s);
      }
    }
  }
  return KVC_ORACLE_OK;
}
