/*
 * kvc.h -- C ABI of the MI355X (gfx950) library for one autoregressive step
 * of a fixed-capacity KV cache: append new key/value rows, then run causal,
 * GQA-aware softmax attention of the step's queries over the updated cache.
 *
 * The operation is the one defined on the page "Autoregressive KV-cache
 * append and causal attention" (biotorch problem kv_cache_attention_step),
 * sections "Function signature", "Required behavior" and "Starter code":
 *
 *   - query head h reads KV head floor(h / (Hq / Hk));
 *   - append_mask[b,:] is a prefix of n_b Trues; new_key/new_value row t is
 *     written to cache slot lengths[b] + t for t < n_b, and the new length
 *     is lengths[b] + n_b;
 *   - valid query t (t < n_b) attends slots j <= lengths[b] + t (and
 *     j < lengths[b] + n_b) -- the lower-right causal alignment fixed by
 *     KempnerForge pull request 542 (Summary);
 *   - scores are scale * dot(q, k), scale > 0, default 1/sqrt(D); the
 *     softmax is taken after subtracting the row maximum;
 *   - attention[B,Hq,Q,M] holds the probabilities (exactly 0 outside the
 *     allowed slots and on invalid rows) and context[B,Hq,Q,Dv] =
 *     attention x updated values (0 on invalid rows);
 *   - every cache entry that is not written keeps its exact bits.
 *
 * Layout.  Every tensor is dense, row-major and contiguous in device memory
 * (HBM), head-major as on the page (and as the continuous cache layout of
 * ClikaRT's attention_over_cache):
 *
 *   query       [B, Hq, Q, D]        new_key     [B, Hk, Q, D]
 *   new_value   [B, Hk, Q, Dv]       key_cache   [B, Hk, M, D]
 *   value_cache [B, Hk, M, Dv]       lengths     [B]  int64
 *   append_mask [B, Q] uint8 (0 = False, other = True)
 *   attention   [B, Hq, Q, M]        context     [B, Hq, Q, Dv]
 *   row_status  [B]  int32 (optional)
 *
 * Floating tensors all have the element type `dtype` (KVC_F32 or KVC_BF16);
 * attention and context are written in that type too.  bf16 inputs are
 * computed with fp32 accumulation; fp32 inputs accumulate scores and softmax
 * statistics in fp64.
 *
 * Ownership.  The caller owns every buffer.  All tensor pointers are device
 * pointers; `dims` and `events` point to host memory.  The library keeps no
 * state between calls, allocates no memory, performs no host/device
 * synchronisation, and enqueues all of its work on `stream` (a hipStream_t;
 * NULL is the default stream).  A call returns once its kernels are
 * enqueued; the outputs are ready when the stream reaches that point.
 * Scratch memory is the caller's `workspace` (size: kvc_workspace_bytes);
 * its contents need no initialisation and are garbage after the call.
 * Calls that share a workspace must be ordered on one stream.
 *
 * Errors.  Argument errors are found on the host before anything is
 * enqueued and returned as a negative KVC_ERR_* code; nothing is written.
 * Rows that break the page's preconditions (length outside [0, M], a mask
 * that is not a prefix, length + n > M) are outside the page's contract;
 * this library treats such a row as a no-op -- its cache row is left (or
 * copied) unchanged, lengths_out[b] = lengths[b], its attention and context
 * are zero -- and reports the reason in row_status[b] (KVC_ROW_*).
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Problem sizes.  B, Hq, Hk, M, D, Dv >= 1; Q >= 0; Hq % Hk == 0. */
typedef struct kvc_dims {
  int64_t B, Hq, Hk, Q, M, D, Dv;
} kvc_dims;

/* Element type of every floating tensor. */
typedef enum kvc_dtype { KVC_F32 = 0, KVC_BF16 = 1 } kvc_dtype;

/* Return codes. */
enum {
  KVC_OK = 0,
  KVC_ERR_NULL = -1,        /* a required pointer is NULL */
  KVC_ERR_SHAPE = -2,       /* sizes out of range, Hq % Hk != 0, or too large */
  KVC_ERR_DTYPE = -3,       /* dtype is not a kvc_dtype */
  KVC_ERR_SCALE = -4,       /* has_scale and scale not finite or <= 0 */
  KVC_ERR_WORKSPACE = -5,   /* workspace_bytes < kvc_workspace_bytes() */
  KVC_ERR_ALIAS = -6,       /* an output overlaps an input or another output */
  KVC_ERR_HIP = -7,         /* a kernel launch failed (HIP error) */
  KVC_ERR_UNSUPPORTED = -8, /* a shape, block size or buffer alignment the entry point does not take */
  KVC_ERR_TOO_LARGE = -9    /* kvc_step_inplace_noalloc: the step needs more than its static scratch */
};

/* Per-row status written to row_status[b]. */
enum {
  KVC_ROW_OK = 0,
  KVC_ROW_BAD_LENGTH = 1,   /* lengths[b] < 0 or > M */
  KVC_ROW_OVERFLOW = 2,     /* lengths[b] + n_b > M */
  KVC_ROW_NOT_PREFIX = 3,   /* append_mask[b,:] has a True after a False */
  KVC_ROW_BAD_QUERIES = 4   /* kvc_attend_over_cache: a sequence's query range is
                               not inside [0, total_q], or holds more than
                               dims->Q tokens or more tokens than are cached */
};

/* Optional timing hook: when a kvc_events is passed, `start` and `stop`
 * (hipEvent_t handles created by the caller) are recorded on the stream
 * immediately before and after the attention kernel of the step. */
typedef struct kvc_events {
  void *start;
  void *stop;
} kvc_events;

/* Kernel plan the library picks for a shape (host-only: it reads the
 * current device's compute-unit count, and assumes 256 without a device). */
typedef struct kvc_plan {
  int32_t path;          /* 0 generic, 1 vector decode, 2 MFMA chunk */
  int32_t rows;          /* packed query rows per KV head: (Hq/Hk) * Q */
  int32_t rows_per_tile; /* packed rows handled by one workgroup */
  int32_t row_tiles;     /* ceil(rows / rows_per_tile) */
  int64_t split;         /* cache slots per split-K workgroup */
  int64_t nsplit;        /* ceil(M / split) */
  size_t workspace_bytes;
  int64_t workers;       /* path 1: decode workers the chunk list is split over */
  int64_t lead;          /* path 1: share weight of the first half of the workers,
                            in eighths (8: even shares) */
} kvc_plan;

/* Bytes of device workspace a step with these sizes needs (0 on bad
 * arguments).  Depends only on dims and dtype. */
size_t kvc_workspace_bytes(const kvc_dims *dims, int dtype);

/* Fill *plan for these sizes; returns KVC_OK or an argument error. */
int kvc_plan_step(const kvc_dims *dims, int dtype, kvc_plan *plan);

/* The page's step, leaving every input untouched ("never modify inputs"):
 * the whole cache is copied bit for bit into key_cache_out/value_cache_out
 * with the new rows in place, lengths_out[b] = lengths[b] + n_b, and
 * attention/context are written.  No output may overlap an input or another
 * output (KVC_ERR_ALIAS).  row_status may be NULL.  With Q = 0 only the
 * cache copy and lengths_out are produced (attention/context may be NULL). */
int kvc_step_out_of_place(const kvc_dims *dims, int dtype, int has_scale,
                          double scale, const void *query,
                          const void *new_key, const void *new_value,
                          const void *key_cache, const void *value_cache,
                          const int64_t *lengths, const uint8_t *append_mask,
                          void *key_cache_out, void *value_cache_out,
                          int64_t *lengths_out, void *attention,
                          void *context, int32_t *row_status, void *workspace,
                          size_t workspace_bytes, void *stream,
                          const kvc_events *events);

/* The same step for production decode: the new rows are written into
 * key_cache/value_cache in place (nothing else of the cache is touched).
 * lengths_out may be the same buffer as lengths (then it is updated in
 * place); any other overlap between outputs, inputs and caches is rejected.
 * With lengths_out != lengths a repeated call repeats the same step. */
int kvc_step_inplace(const kvc_dims *dims, int dtype, int has_scale,
                     double scale, const void *query, const void *new_key,
                     const void *new_value, void *key_cache, void *value_cache,
                     const int64_t *lengths, const uint8_t *append_mask,
                     int64_t *lengths_out, void *attention, void *context,
                     int32_t *row_status, void *workspace,
                     size_t workspace_bytes, void *stream,
                     const kvc_events *events);

/* The same in-place step over a paged cache -- the block-pool layout that
 * ClikaRT's attention_over_cache names beside the continuous one (a pool
 * [num_blocks, H_kv, block_size, D] with a rank-2 [B, max_blocks] block
 * table):
 *
 *   key_pool    [num_blocks, Hk, block_size, D]
 *   value_pool  [num_blocks, Hk, block_size, Dv]
 *   block_table [B, M / block_size] int32
 *
 * Slot j of batch row b -- key_cache[b, h, j, :] of the dense layout -- is
 * key_pool[block_table[b, j / block_size], h, j % block_size, :] (the same
 * for values).  dims->M is each row's capacity and a multiple of
 * block_size; everything else (lengths, mask, query, new rows, attention,
 * context, row_status, workspace) is as for kvc_step_inplace, and the
 * results equal kvc_step_inplace's on the dense cache the table describes.
 *
 * block_size: a power of two that divides M, or M itself (one block per
 * row: a continuous cache whose rows the table picks); else KVC_ERR_SHAPE.
 * Every shape of kvc_step_inplace is taken: the vector decode and
 * matrix-core chunk paths read the pools when the buffers are 16-byte
 * aligned and each of their chunks (64 slots) sits in one block; other
 * calls (smaller blocks, misaligned pools, head sizes without those
 * kernels) take the generic kernel.  Table entries are device data: an entry outside
 * [0, num_blocks) for a slot below lengths[b] + n_b is outside the contract
 * -- those slots read as zero rows and are never written, so no access
 * leaves the pools -- and the row's results are then unspecified.  Rows may
 * share blocks for slots below their lengths (a shared prefix); a block that
 * receives appended rows must not be used by another row of the same step.
 * The pools, the table and every other input must not overlap the outputs
 * (KVC_ERR_ALIAS); lengths_out may be lengths. */
int kvc_step_paged(const kvc_dims *dims, int dtype, int has_scale,
                   double scale, const void *query, const void *new_key,
                   const void *new_value, void *key_pool, void *value_pool,
                   int64_t num_blocks, int64_t block_size,
                   const int32_t *block_table, const int64_t *lengths,
                   const uint8_t *append_mask, int64_t *lengths_out,
                   void *attention, void *context, int32_t *row_status,
                   void *workspace, size_t workspace_bytes, void *stream,
                   const kvc_events *events);

/* Read-only re-attention over a cache another call already appended
 * ("ClikaRT::ops::attention_over_cache", function description): no cache
 * entry is written.
 *
 *   q            [total_q, Hq, D]   packed varlen queries; sequence b owns
 *                                   rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   cu_seqlens_q [B + 1] int64      (S_b = cu_seqlens_q[b+1] - cu_seqlens_q[b])
 *   seqlens_k    int64, seqlens_k_count entries: each sequence's total
 *                cached length L_b, either per sequence ([B]: L_b =
 *                seqlens_k[b]) or cumulative ([B + 1]: L_b = seqlens_k[b+1]
 *                - seqlens_k[b]) -- the page's two forms of cu_seqlens_k;
 *                any other count is KVC_ERR_SHAPE
 *   head_sink    [Hq] float32       optional per-head sink logit
 *   out          [total_q, Hq, Dv]  written for every query row
 *
 * The cache is one of three layouts:
 *   - paged: block_table [B, M / block_size] int32 (slot_ids NULL), pools
 *     [num_blocks, Hk, block_size, D|Dv] as for kvc_step_paged;
 *   - continuous with slot_ids [B] int32 (block_table NULL): key_cache
 *     [num_blocks, Hk, M, D], sequence b reading row slot_ids[b];
 *   - continuous without either: sequence b reads row b (num_blocks >= B).
 * block_size is M (or 0) for the continuous layouts.
 *
 * dims: B sequences, Hq, Hk, Q = the most query tokens any sequence has,
 * M = capacity per sequence, D, Dv.  Query t of sequence b sits at position
 * L_b - S_b + t and attends slots j <= L_b - S_b + t (the lower-right
 * alignment of the step); scores are scale * dot(q, k) (default 1/sqrt(D)),
 * and the softmax denominator gains exp(head_sink[h] - m) when a sink is
 * given (the sink is a logit on the scores' scale and carries no value).
 * A sequence with L_b outside [0, M] (KVC_ROW_BAD_LENGTH) or a bad query
 * range (KVC_ROW_BAD_QUERIES) gets zero output rows where its range is
 * addressable, and its code in row_status (optional).
 *
 * Scope: every shape of kvc_step_inplace, in each layout (the paged one
 * with kvc_step_paged's block sizes).
 * workspace: kvc_attend_workspace_bytes(dims, dtype) bytes.  Outputs and the
 * workspace must not overlap any input (KVC_ERR_ALIAS). */
size_t kvc_attend_workspace_bytes(const kvc_dims *dims, int dtype);
int kvc_attend_over_cache(const kvc_dims *dims, int dtype, int has_scale,
                          double scale, const void *q, int64_t total_q,
                          const int64_t *cu_seqlens_q, const void *key_cache,
                          const void *value_cache, int64_t num_blocks,
                          int64_t block_size, const int32_t *block_table,
                          const int32_t *slot_ids, const int64_t *seqlens_k,
                          int64_t seqlens_k_count, const float *head_sink, void *out,
                          int32_t *row_status, void *workspace,
                          size_t workspace_bytes, void *stream,
                          const kvc_events *events);

/* Backward of the step (fp32 or bf16: every tensor argument of the dtype,
 * gradients in and out included; any head sizes with D + Dv <= 6144; every
 * buffer aligned to its element; else KVC_ERR_UNSUPPORTED): the gradients
 * of the step's inputs given those of its outputs.  Head sizes (64, 64),
 * (128, 128) and (64, 32) with query, key_cache, value_cache, new_key,
 * new_value, d_context, d_key_cache_out, d_value_cache_out and the five
 * gradient outputs 16-byte aligned take tiled kernels (and bf16 heads of
 * at most 8 packed rows with D = Dv in {64, 128} vector-unit ones); every
 * other call takes generic kernels with scalar loads, in fp64 throughout.
 * The math runs in fp32 and fp64 either way; each gradient is rounded once
 * to the dtype.  The page grades gradients as well as values
 * ("Autoregressive KV-cache append and causal attention", the workspace
 * note).
 *
 * Inputs: the step's own inputs (query, new_key, new_value, lengths,
 * append_mask as given to the step; key_cache / value_cache either the
 * caches before the step or after an in-place step -- only slots below
 * lengths[b] are read from them) and the gradients of its outputs
 * d_attention [B,Hq,Q,M], d_context [B,Hq,Q,Dv], d_key_cache_out
 * [B,Hk,M,D], d_value_cache_out [B,Hk,M,Dv] (each may be NULL = zero).
 * The attention is recomputed from the scores with fp64 row statistics,
 * so the forward's outputs are not needed.
 * Outputs (all written): g_query [B,Hq,Q,D], g_new_key [B,Hk,Q,D],
 * g_new_value [B,Hk,Q,Dv], g_key_cache [B,Hk,M,D], g_value_cache
 * [B,Hk,M,Dv].  With K', V' the updated caches and P the attention of a
 * valid row (t < n_b): dP_j = dA_j + dO.V'_j on j <= lengths[b] + t,
 * dS_j = P_j (dP_j - sum_k P_k dP_k), g_query = scale sum_j dS_j K'_j,
 * dK'_j gains scale dS_j q and dV'_j gains P_j dO; dK' plus the returned
 * cache's gradient goes to g_key_cache at kept slots and to g_new_key at
 * the appended slots (whose old cache entries get 0).  Tokens t >= n_b and
 * rows outside the contract get zero query and new-row gradients; their
 * cache passes its gradient through.
 * workspace: kvc_backward_workspace_bytes(dims, dtype) bytes.  No output
 * may overlap an input or another output (KVC_ERR_ALIAS). */
size_t kvc_backward_workspace_bytes(const kvc_dims *dims, int dtype);
int kvc_step_backward(const kvc_dims *dims, int dtype, int has_scale,
                      double scale, const void *query, const void *new_key,
                      const void *new_value, const void *key_cache,
                      const void *value_cache, const int64_t *lengths,
                      const uint8_t *append_mask, const void *d_attention,
                      const void *d_context, const void *d_key_cache_out,
                      const void *d_value_cache_out, void *g_query,
                      void *g_new_key, void *g_new_value, void *g_key_cache,
                      void *g_value_cache, void *workspace,
                      size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as kvc_step_inplace, with the same arguments minus the workspace.
 * Its workspace is a static device array inside the library, of
 * kvc_noalloc_scratch_bytes() bytes (96 MiB) on every GPU the library runs
 * on, held until the process ends.  A step whose kvc_workspace_bytes()
 * exceeds it returns KVC_ERR_TOO_LARGE before anything is enqueued.  The
 * call allocates nothing: on its first use on a device it looks up that
 * device's copy of the array (hipGetSymbolAddress) and keeps the address.
 * Every call on one GPU shares that array, and nothing in it needs to start
 * at any value; calls that overlap on one GPU (two streams, or two host
 * threads without ordering) race on it -- order them on one stream. */
size_t kvc_noalloc_scratch_bytes(void);
int kvc_step_inplace_noalloc(const kvc_dims *dims, int dtype, int has_scale,
                             double scale, const void *query,
                             const void *new_key, const void *new_value,
                             void *key_cache, void *value_cache,
                             const int64_t *lengths,
                             const uint8_t *append_mask, int64_t *lengths_out,
                             void *attention, void *context,
                             int32_t *row_status, void *stream,
                             const kvc_events *events);

/* Static description of a return or row-status code. */
const char *kvc_status_string(int code);

/* Measurement helper (no part of the step): stream-reads `bytes` of the
 * device buffer `buffer` with the non-temporal 16-byte loads the attend
 * kernels use for K/V rows, one contiguous slab per workgroup, and folds
 * what each lane read into one word of `sink` (a device buffer of at least
 * kvc_read_ceiling_sink_bytes(workgroups) bytes) so that no load is dead.
 * `bytes` must be a multiple of workgroups * 32 KiB (else KVC_ERR_SHAPE).
 * Enqueued on `stream`; time it with events around the call to get an
 * achievable read bandwidth of the part. */
size_t kvc_read_ceiling_sink_bytes(int workgroups);
int kvc_read_ceiling(const void *buffer, size_t bytes, int workgroups,
                     void *sink, size_t sink_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
