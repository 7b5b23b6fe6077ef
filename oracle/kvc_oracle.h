/*
 * kvc_oracle.h -- plain CPU reference of one KV-cache append + causal GQA
 * attention step, in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library
 * against the definition of the step.  Only the test-suite, the smoke check
 * and the CPU-baseline leg of the benchmark load it.  The product library
 * never links it, includes it or calls it, and it shares no source with it.
 *
 * The operation follows the page "Autoregressive KV-cache append and causal
 * attention" (biotorch, problem kv_cache_attention_step), section "Required
 * behavior".  All tensors are dense, row-major, host memory:
 *
 *   query       [B, Hq, Q, D]      new_key   [B, Hk, Q, D]
 *   new_value   [B, Hk, Q, Dv]     key_cache [B, Hk, M, D]
 *   value_cache [B, Hk, M, Dv]     lengths   [B]  int64
 *   append_mask [B, Q]  uint8 (0 = False, anything else = True)
 *
 * Element type: dtype 0 = IEEE binary32, dtype 1 = bfloat16 (raw 16-bit
 * words).  Both widen exactly to double; every sum, max, exp and division
 * below is done in double.
 */
#ifndef KVC_ORACLE_H
#define KVC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes (negative = argument error, nothing written). */
#define KVC_ORACLE_OK 0
#define KVC_ORACLE_ESHAPE (-1)
#define KVC_ORACLE_ESCALE (-2)
#define KVC_ORACLE_EDTYPE (-3)
#define KVC_ORACLE_ENULL (-4)

/* Per-row status codes written to row_status[b]; a row with a non-zero
 * status is left unchanged (the reading of the outside-contract cases). */
#define KVC_ORACLE_ROW_OK 0
#define KVC_ORACLE_ROW_BAD_LENGTH 1
#define KVC_ORACLE_ROW_OVERFLOW 2
#define KVC_ORACLE_ROW_NOT_PREFIX 3
#define KVC_ORACLE_ROW_BAD_QUERIES 4

/* Append only: copies both caches bit for bit into *_out, writes the True
 * prefix of new rows at slots length+t, and returns lengths_out, the number
 * of appended rows n_out[b] (0 on a rejected row) and row_status[b]. */
int kvc_oracle_append(int64_t B, int64_t Hq, int64_t Hk, int64_t Q, int64_t M,
                      int64_t D, int64_t Dv, int dtype,
                      const void *new_key, const void *new_value,
                      const void *key_cache, const void *value_cache,
                      const int64_t *lengths, const uint8_t *append_mask,
                      void *key_cache_out, void *value_cache_out,
                      int64_t *lengths_out, int64_t *n_out,
                      int32_t *row_status);

/* One query row (b, hq, t) over an already-updated cache whose old length
 * was old_len and which received n rows.  Writes attention_row[M] and
 * context_row[Dv] (zeros when t >= n).  has_scale = 0 selects 1/sqrt(D). */
int kvc_oracle_attend_row(int64_t B, int64_t Hq, int64_t Hk, int64_t Q,
                          int64_t M, int64_t D, int64_t Dv, int dtype,
                          int has_scale, double scale, const void *query,
                          const void *key_updated, const void *value_updated,
                          int64_t old_len, int64_t n, int64_t b, int64_t hq,
                          int64_t t, double *attention_row,
                          double *context_row);

/* The whole step: append, then every (b, hq, t) row.
 * attention [B, Hq, Q, M] and context [B, Hq, Q, Dv] are double. */
int kvc_oracle_step(int64_t B, int64_t Hq, int64_t Hk, int64_t Q, int64_t M,
                    int64_t D, int64_t Dv, int dtype, int has_scale,
                    double scale, const void *query, const void *new_key,
                    const void *new_value, const void *key_cache,
                    const void *value_cache, const int64_t *lengths,
                    const uint8_t *append_mask, void *key_cache_out,
                    void *value_cache_out, int64_t *lengths_out,
                    double *attention, double *context, int32_t *row_status);

/* Read-only re-attention over an already-appended cache ("ClikaRT::ops::
 * attention_over_cache", function description): packed varlen queries
 * q [Tq, Hq, D], sequence b owning rows cu_q[b] .. cu_q[b+1]-1 (S_b of
 * them), over the logical cache key [B, Hk, M, D] / value [B, Hk, M, Dv]
 * of which seqlens_k[b] = L_b slots are filled.  Query t of sequence b sits
 * at position L_b - S_b + t and attends slots j <= L_b - S_b + t.  sink
 * (double [Hq], or NULL) is a virtual logit per query head added to the
 * softmax denominator.  out [Tq, Hq, Dv] double; status[b]:
 * KVC_ORACLE_ROW_BAD_LENGTH (L_b outside [0, M]) or
 * KVC_ORACLE_ROW_BAD_QUERIES (S_b < 0, S_b > Q or S_b > L_b), whose rows
 * are zero. */
int kvc_oracle_reattend(int64_t B, int64_t Hq, int64_t Hk, int64_t Q,
                        int64_t M, int64_t D, int64_t Dv, int dtype,
                        int has_scale, double scale, int64_t Tq,
                        const void *q, const int64_t *cu_q, const void *key,
                        const void *value, const int64_t *seqlens_k,
                        const double *sink, double *out, int32_t *status);

#ifdef __cplusplus
}
#endif

#endif
