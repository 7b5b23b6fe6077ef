// kvc_reattend.h -- read-only re-attention over a cache another call has
// already appended ("ClikaRT::ops::attention_over_cache", function
// description): packed varlen queries q [Tq, Hq, D], sequence b owning rows
// cu_q[b] .. cu_q[b+1]-1 (S_b of them) and seqlens_k[b] = L_b cached
// slots.  Query t of sequence b sits at position L_b - S_b + t, so it sees
// slots j <= L_b - S_b + t: exactly the step whose old length is L_b - S_b
// and whose S_b appended rows are the cache's rows [L_b - S_b, L_b).  The
// two kernels here turn the request into that step (run by the stream or
// chunk kernels in read-only mode, with the per-head sink added by the
// combine kernel) and scatter its context back to the packed layout.
#pragma once

#include "kvc_common.h"
#include "kvc_generic.h"

namespace kvc {

constexpr int kReattThreads = 256;
// row status codes (include/kvc.h, KVC_ROW_*)
constexpr int32_t kRowOk = 0, kRowBadLength = 1, kRowBadQueries = 4;

struct ReattArgs {
  int64_t Tq;
  const uint8_t* q;          // [Tq][Hq][D]
  const int64_t* cu_q;       // [B + 1]
  const int64_t* seqlens_k;  // [B]
  uint8_t* out;              // [Tq][Hq][Dv]
  int32_t* row_status;       // [B] or null
  // the equivalent step's inputs and context, in the workspace
  int64_t* len0;   // [B]: L - S
  uint8_t* mask;   // [B][Q]
  uint8_t* qs;     // [B][Hq][Q][D]
  uint8_t* nk;     // [B][Hk][Q][D]
  uint8_t* nv;     // [B][Hk][Q][Dv]
  int32_t* rstat;  // [B]
  const uint8_t* ctx;  // [B][Hq][Q][Dv]
};

// Row checks of sequence b: a cached length outside [0, M] (bad length), or
// a query range that is not inside [0, Tq], holds more than Q tokens or more
// tokens than are cached (bad queries).
__device__ inline int32_t reatt_status(const StepArgs& a, const ReattArgs& r, int64_t b) {
  const int64_t L = r.seqlens_k[b], c0 = r.cu_q[b], c1 = r.cu_q[b + 1], S = c1 - c0;
  if (L < 0 || L > a.M) return kRowBadLength;
  if (c0 < 0 || c1 > r.Tq || S < 0 || S > a.Q || S > L) return kRowBadQueries;
  return kRowOk;
}

// One workgroup per sequence: the step's old length, mask and query rows,
// and the S cache rows [L - S, L) of every KV head as its "appended" rows
// (through the same slot mapping the attend kernel uses; a slot outside
// the pool reads as zeros).
__global__ __launch_bounds__(kReattThreads) void reattend_prep_kernel(StepArgs a, ReattArgs r) {
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t st = reatt_status(a, r, b);
  const bool ok = st == kRowOk;
  const int64_t L = r.seqlens_k[b], c0 = r.cu_q[b], S = ok ? r.cu_q[b + 1] - c0 : 0;
  if (tid == 0) {
    r.len0[b] = ok ? L - S : 0;
    r.rstat[b] = st;
  }
  for (int64_t t = tid; t < a.Q; t += kReattThreads) r.mask[b * a.Q + t] = t < S ? 1 : 0;
  const int64_t e = a.elem_bytes, qb = a.D * e, kb = a.D * e, vb = a.Dv * e;
  for (int64_t i = 0; i < S * a.Hq; i++) {
    const int64_t t = i / a.Hq, hq = i % a.Hq;
    copy_bytes(r.qs + ((b * a.Hq + hq) * a.Q + t) * qb, r.q + ((c0 + t) * a.Hq + hq) * qb, qb,
               tid, kReattThreads);
  }
  for (int64_t i = 0; i < S * a.Hk; i++) {
    const int64_t t = i / a.Hk, h = i % a.Hk, j = L - S + t;
    uint8_t* kd = r.nk + ((b * a.Hk + h) * a.Q + t) * kb;
    uint8_t* vd = r.nv + ((b * a.Hk + h) * a.Q + t) * vb;
    const uint8_t* ks = slot_row(a, a.kc_in, b, h, j, kb);
    const uint8_t* vs = slot_row(a, a.vc_in, b, h, j, vb);
    if (ks) {
      copy_bytes(kd, ks, kb, tid, kReattThreads);
    } else {
      for (int64_t x = tid; x < kb; x += kReattThreads) kd[x] = 0;
    }
    if (vs) {
      copy_bytes(vd, vs, vb, tid, kReattThreads);
    } else {
      for (int64_t x = tid; x < vb; x += kReattThreads) vd[x] = 0;
    }
  }
}

// One workgroup per sequence: its context rows to the packed output (zeros
// for a rejected sequence whose query range is addressable), and its status.
__global__ __launch_bounds__(kReattThreads) void reattend_scatter_kernel(StepArgs a,
                                                                         ReattArgs r) {
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t st = r.rstat[b];
  if (tid == 0 && r.row_status) r.row_status[b] = st;
  const int64_t c0 = r.cu_q[b], c1 = r.cu_q[b + 1], S = c1 - c0;
  if (c0 < 0 || c1 > r.Tq || S <= 0) return;
  const int64_t vb = a.Dv * a.elem_bytes;
  for (int64_t i = 0; i < S * a.Hq; i++) {
    const int64_t t = i / a.Hq, hq = i % a.Hq;
    uint8_t* dst = r.out + ((c0 + t) * a.Hq + hq) * vb;
    if (st == kRowOk) {
      copy_bytes(dst, r.ctx + ((b * a.Hq + hq) * a.Q + t) * vb, vb, tid, kReattThreads);
    } else {
      for (int64_t x = tid; x < vb; x += kReattThreads) dst[x] = 0;
    }
  }
}

}  // namespace kvc
