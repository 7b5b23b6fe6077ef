// kvc_prep.h -- row preparation for the stream-mode attend kernel.
//
// One workgroup computes, for every batch row b, the row information of
// "Autoregressive KV-cache append and causal attention" (Required
// behavior: n = count of the True prefix of append_mask[b,:], 0 <= length
// <= M, length + n <= M; a broken row becomes a no-op with a status), the
// number of C-slot chunks each of its KV heads needs, and the exclusive
// prefix sum of Hk * chunks over b (the row's first index in the flattened
// chunk list).  Its output is all the attend and combine kernels read about
// lengths and masks, so lengths_out may alias lengths.
#pragma once

#include "kvc_common.h"

namespace kvc {

constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(StepArgs a) {
  __shared__ int64_t wave_total[kPrepThreads / kWave];
  __shared__ int64_t carry_sh;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  if (tid == 0) carry_sh = 0;
  __syncthreads();
  for (int64_t base = 0; base < a.B; base += kPrepThreads) {
    const int64_t b = base + tid;
    RowInfo ri{0, 0, 0};
    int64_t chunks = 0;
    if (b < a.B) {
      ri = thread_row_info(a.lengths, a.mask, a.Q, a.M, b);
      chunks = a.Hk * row_chunks(ri.len, ri.n, a.C);
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
    }
    __syncthreads();
    if (tid == kPrepThreads - 1) carry_sh = before + incl;
    __syncthreads();
  }
  if (tid == 0) a.ws_hdr[0] = carry_sh;
}

}  // namespace kvc
