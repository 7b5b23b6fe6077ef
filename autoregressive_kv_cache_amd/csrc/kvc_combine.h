// kvc_combine.h -- merge of split-K partial results by log-sum-exp.
//
// For a packed query row with split statistics (m_s, l_s, o_s):
//   m = max_s m_s,  l = sum_s l_s exp(m_s - m),
//   context = sum_s o_s exp(m_s - m) / l,
// and the probabilities exp(s_j - m_s) that the split kernel left in the
// attention buffer become exp(s_j - m) / l after one multiplication by
// exp(m_s - m) / l -- the normalised softmax of "Autoregressive KV-cache
// append and causal attention" (Required behavior).  The kernel also writes
// lengths_out and row_status, reading the row information the split kernel
// published (never `lengths` itself, which lengths_out may alias).
//
// Grid: one workgroup per (b, KV head, split), the same flattening as the
// split kernels.  Every workgroup rescales the attention of its own split
// for all rows of its KV head; the context of row r is reduced by the
// workgroup of split (r mod active splits).
#pragma once

#include "kvc_common.h"

namespace kvc {

constexpr int kCombineThreads = 256;

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(StepArgs a) {
  using E = Elem<T>;
  using Acc = typename E::Acc;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t s = blockIdx.x % a.nsplit;
  const int64_t grp = blockIdx.x / a.nsplit;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;
  const int64_t len = a.ws_rowinfo[b * 4 + 0];
  const int64_t n = a.ws_rowinfo[b * 4 + 1];
  const int32_t status = static_cast<int32_t>(a.ws_rowinfo[b * 4 + 2]);

  if (s == 0 && kvh == 0 && tid == 0) {
    a.lengths_out[b] = len + n;
    if (a.row_status) a.row_status[b] = status;
  }
  const int64_t nsa = active_splits(len, n, a.S);
  if (nsa <= 1 || s >= nsa) return;

  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  const int64_t s0 = s * a.S;
  T* att = static_cast<T*>(a.attention);
  T* ctx = static_cast<T*>(a.context);
  const double* ml_grp = a.ws_ml + grp * a.nsplit * a.R * 2;
  const float* o_grp = a.ws_o + grp * a.nsplit * a.R * a.Dv;

  for (int r = wave; r < a.R; r += kCombineThreads / kWave) {
    const int64_t g = r / a.Q, t = r % a.Q;
    const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
    const bool ctx_owner = (r % nsa) == s;
    if (t >= n) {  // invalid row: attention already zero; context zero
      if (ctx_owner)
        for (int64_t dv = lane; dv < a.Dv; dv += kWave) ctx[row * a.Dv + dv] = E::zero();
      continue;
    }
    Acc m = neg_inf;
    for (int64_t k = lane; k < nsa; k += kWave) {
      const Acc mk = static_cast<Acc>(ml_grp[(k * a.R + r) * 2]);
      m = mk > m ? mk : m;
    }
    m = wave_max(m);
    Acc l = 0;
    for (int64_t k = lane; k < nsa; k += kWave) {
      const Acc mk = static_cast<Acc>(ml_grp[(k * a.R + r) * 2]);
      if (mk != neg_inf) l += static_cast<Acc>(ml_grp[(k * a.R + r) * 2 + 1]) * acc_exp(mk - m);
    }
    l = wave_sum(l);
    const Acc inv_l = Acc(1) / l;

    // rescale this split's probabilities of row r
    const Acc ms = static_cast<Acc>(ml_grp[(s * a.R + r) * 2]);
    const Acc f = ms == neg_inf ? Acc(0) : acc_exp(ms - m) * inv_l;
    const int64_t last = len + t;  // last visible slot
    const int64_t e1 = (s0 + a.S < last + 1) ? s0 + a.S : last + 1;
    T* arow = att + row * a.M;
    for (int64_t j = s0 + lane; j < e1; j += kWave) E::store(arow + j, E::load(arow + j) * f);

    if (ctx_owner) {
      for (int64_t dv = lane; dv < a.Dv; dv += kWave) {
        Acc o = 0;
        for (int64_t k = 0; k < nsa; k++) {
          const Acc mk = static_cast<Acc>(ml_grp[(k * a.R + r) * 2]);
          if (mk == neg_inf) continue;
          o += static_cast<Acc>(o_grp[(k * a.R + r) * a.Dv + dv]) * acc_exp(mk - m);
        }
        E::store(ctx + row * a.Dv + dv, o * inv_l);
      }
    }
  }
}

}  // namespace kvc
