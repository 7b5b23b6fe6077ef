// kvc_prep.h -- row preparation for the stream path on large batches.
//
// One workgroup works out every batch row's information as "Autoregressive
// KV-cache append and causal attention" (Required behavior) defines it --
// n = count of the True prefix of append_mask[b,:], 0 <= length <= M,
// length + n <= M; a broken row becomes a no-op with a status -- the number
// of stream chunks each KV head needs (stream_chunks), the exclusive prefix
// sum of Hk * chunks over b (each row's first index in the flattened chunk
// list), the number of busy stream workers Pe = min(P, Nc), and each
// worker's first chunk.  (Batches of up to kDecodeFusedRows rows skip this
// kernel: the attend kernel builds the same table in LDS.)
//
// After this kernel the attend and combine kernels read row information
// only from the workspace, so lengths_out may alias lengths.
#pragma once

#include "kvc_common.h"

namespace kvc {

constexpr int kPrepThreads = 1024;
constexpr int kPrepLdsRows = 2048;  // rows whose first-chunk index stays in LDS

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(StepArgs a) {
  __shared__ int64_t wave_total[kPrepThreads / kWave];
  __shared__ int64_t first_sh[kPrepLdsRows];
  __shared__ int32_t nc_sh[kPrepLdsRows];
  __shared__ int64_t carry_sh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  // ---- row information, chunk offsets and worker starts ----
  if (tid == 0) carry_sh = 0;
  __syncthreads();
  for (int64_t base = 0; base < a.B; base += kPrepThreads) {
    const int64_t b = base + tid;
    RowInfo ri{0, 0, 0};
    int64_t chunks = 0;
    if (b < a.B) {
      ri = thread_row_info(a.lengths, a.mask, a.Q, a.M, b);
      chunks = a.Hk * stream_chunks(ri.len, ri.n, a.C);
    }
    // inclusive scan inside the wave
    int64_t incl = chunks;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int64_t up = __shfl_up(incl, o);
      if (lane >= o) incl += up;
    }
    if (lane == kWave - 1) wave_total[wave] = incl;
    __syncthreads();
    int64_t before = carry_sh;
    for (int k = 0; k < wave; k++) before += wave_total[k];
    if (b < a.B) {
      int64_t* row = a.ws_rowinfo + b * 4;
      row[0] = ri.len;
      row[1] = ri.n;
      row[2] = ri.status;
      row[3] = before + incl - chunks;
      if (b < kPrepLdsRows) {
        first_sh[b] = before + incl - chunks;
        nc_sh[b] = static_cast<int32_t>(stream_chunks(ri.len, ri.n, a.C));
      }
    }
    __syncthreads();
    if (tid == kPrepThreads - 1) carry_sh = before + incl;
    __syncthreads();
  }
  const int64_t Nc = carry_sh;
  // stream workers that get work: at most one per chunk, so that every one
  // of them owns at least one chunk
  const int64_t Pe = Nc < a.P ? (Nc > 0 ? Nc : 1) : a.P;
  if (tid == 0) {
    a.ws_hdr[0] = Nc;
    a.ws_hdr[1] = Pe;
  }
  if (Nc == 0) return;
  const int32_t lead = effective_lead(Nc, Pe, a.lead);
  // first chunk of each worker: x = worker_start(w) -> (b, head, chunk);
  // the search reads the row starts from LDS when they all fit there
  const bool in_lds = a.B <= kPrepLdsRows;
  for (int64_t wk = tid; wk < Pe; wk += kPrepThreads) {
    const int64_t x = worker_start(wk, Nc, Pe, lead);
    int64_t lo = 0, hi = a.B - 1;  // last row whose first chunk index <= x
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      const int64_t first = in_lds ? first_sh[mid] : a.ws_rowinfo[mid * 4 + 3];
      if (first <= x) lo = mid; else hi = mid - 1;
    }
    const int64_t nc = in_lds ? nc_sh[lo]
                              : stream_chunks(a.ws_rowinfo[lo * 4 + 0], a.ws_rowinfo[lo * 4 + 1], a.C);
    const int64_t rel = x - (in_lds ? first_sh[lo] : a.ws_rowinfo[lo * 4 + 3]);
    int32_t* ws = a.ws_wstart + wk * 4;
    ws[0] = static_cast<int32_t>(lo);
    ws[1] = static_cast<int32_t>(rel / nc);
    ws[2] = static_cast<int32_t>(rel % nc);
    ws[3] = 0;
  }
}

}  // namespace kvc
