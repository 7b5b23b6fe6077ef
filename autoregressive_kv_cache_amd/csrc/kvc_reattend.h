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
  const int64_t* seqlens_k;  // [B] lengths, or [B + 1] cumulative offsets (cum_k)
  int32_t cum_k;
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

// Copy `rows` rows of `rb` bytes, row i from src(i) to dst(i) (null src:
// zeros), all rows at once: 16-byte pieces over the whole workgroup when
// every address and the row size allow it, else 2-byte ones.
template <typename Src, typename Dst>
__device__ inline void copy_rows(int64_t rows, int64_t rb, Src src, Dst dst, bool aligned16) {
  const int tid = threadIdx.x;
  if (aligned16 && rb % 16 == 0) {
    const int64_t parts = rb / 16;
    for (int64_t i = tid; i < rows * parts; i += kReattThreads) {
      const int64_t row = i / parts, part = i % parts;
      const uint8_t* sp = src(row);
      const uint4 v = sp ? reinterpret_cast<const uint4*>(sp)[part] : make_uint4(0, 0, 0, 0);
      reinterpret_cast<uint4*>(dst(row))[part] = v;
    }
  } else {
    const int64_t parts = rb / 2;
    for (int64_t i = tid; i < rows * parts; i += kReattThreads) {
      const int64_t row = i / parts, part = i % parts;
      const uint8_t* sp = src(row);
      const uint16_t v = sp ? reinterpret_cast<const uint16_t*>(sp)[part] : uint16_t(0);
      reinterpret_cast<uint16_t*>(dst(row))[part] = v;
    }
  }
}

// Sequence b's total cached length L_b: seqlens_k[b], or seqlens_k[b + 1] -
// seqlens_k[b] in the cumulative form ("ClikaRT::ops::attention_over_cache",
// function description: per-seq [B] or cumulative [B+1]).
__device__ inline int64_t reatt_len(const ReattArgs& r, int64_t b) {
  return r.cum_k ? r.seqlens_k[b + 1] - r.seqlens_k[b] : r.seqlens_k[b];
}

// Row checks of sequence b: a cached length outside [0, M] (bad length), or
// a query range that is not inside [0, Tq], holds more than Q tokens or more
// tokens than are cached (bad queries).
__device__ inline int32_t reatt_status(const StepArgs& a, const ReattArgs& r, int64_t b) {
  const int64_t L = reatt_len(r, b), c0 = r.cu_q[b], c1 = r.cu_q[b + 1], S = c1 - c0;
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
  const int64_t L = reatt_len(r, b), c0 = r.cu_q[b], S = ok ? r.cu_q[b + 1] - c0 : 0;
  if (tid == 0) {
    r.len0[b] = ok ? L - S : 0;
    r.rstat[b] = st;
  }
  for (int64_t t = tid; t < a.Q; t += kReattThreads) r.mask[b * a.Q + t] = t < S ? 1 : 0;
  const int64_t e = a.elem_bytes, qb = a.D * e, kb = a.D * e, vb = a.Dv * e;
  const bool al = ((reinterpret_cast<uintptr_t>(r.q) | reinterpret_cast<uintptr_t>(a.kc_in) |
                    reinterpret_cast<uintptr_t>(a.vc_in) | reinterpret_cast<uintptr_t>(r.qs) |
                    reinterpret_cast<uintptr_t>(r.nk) | reinterpret_cast<uintptr_t>(r.nv)) & 15u) == 0;
  // query row (t, hq) -> step query (b, hq, t)
  copy_rows(
      S * a.Hq, qb, [&](int64_t i) { return r.q + ((c0 + i / a.Hq) * a.Hq + i % a.Hq) * qb; },
      [&](int64_t i) { return r.qs + ((b * a.Hq + i % a.Hq) * a.Q + i / a.Hq) * qb; }, al);
  // cache row L - S + t of head h -> the step's appended row (b, h, t)
  copy_rows(
      S * a.Hk, kb,
      [&](int64_t i) { return slot_row(a, a.kc_in, b, i % a.Hk, L - S + i / a.Hk, kb); },
      [&](int64_t i) { return r.nk + ((b * a.Hk + i % a.Hk) * a.Q + i / a.Hk) * kb; }, al);
  copy_rows(
      S * a.Hk, vb,
      [&](int64_t i) { return slot_row(a, a.vc_in, b, i % a.Hk, L - S + i / a.Hk, vb); },
      [&](int64_t i) { return r.nv + ((b * a.Hk + i % a.Hk) * a.Q + i / a.Hk) * vb; }, al);
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
  const bool al = ((reinterpret_cast<uintptr_t>(r.out) | reinterpret_cast<uintptr_t>(r.ctx)) &
                   15u) == 0;
  const bool ok = st == kRowOk;
  copy_rows(
      S * a.Hq, vb,
      [&](int64_t i) -> const uint8_t* {
        return ok ? r.ctx + ((b * a.Hq + i % a.Hq) * a.Q + i / a.Hq) * vb : nullptr;
      },
      [&](int64_t i) { return r.out + ((c0 + i / a.Hq) * a.Hq + i % a.Hq) * vb; }, al);
}

}  // namespace kvc
