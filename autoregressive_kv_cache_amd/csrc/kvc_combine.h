// kvc_combine.h -- log-sum-exp merge of the chunk/segment results and the
// final writes of the step.
//
// For a valid packed query row with segment statistics (m_seg, l_seg, o_seg):
//   m = max m_seg,  l = sum l_seg exp(m_seg - m),
//   context = sum o_seg exp(m_seg - m) / l,
// and the values exp(s_j - m_c) the attend kernel left in the attention
// buffer become exp(s_j - m) / l after one multiplication by
// exp(m_c - m) / l -- the normalised softmax of "Autoregressive KV-cache
// append and causal attention" (Required behavior).  Slots after
// length + t and whole invalid rows get exact zeros.
//
// Grid: one workgroup per (b, KV head, range k of CS slots) over all
// ceil(M / CS) ranges, so the zero tails are written by the same dense
// pass.  The context of packed row r is reduced by the workgroup of range
// r mod ceil(M / CS), and the one of (b, head 0, range 0) writes
// lengths_out[b] and row_status[b] from the row
// information the attend side published (never from `lengths`, which
// lengths_out may alias).  In stream mode, out of place, it also copies the
// cache slots the attend kernel did not visit (slots >= length + n, or the
// whole row when n = 0), bit for bit.
#pragma once

#include "kvc_common.h"
#include "kvc_generic.h"

namespace kvc {

constexpr int kCombineThreads = 256;

// Segment ids of group g in stream mode: the workers w whose chunk range
// [start(w), start(w+1)) meets the group's chunks [x0, x1].
struct StreamSegs {
  int64_t Nc, P, x0, x1, g;
  __device__ int64_t start(int64_t w) const { return w * Nc / P; }
  __device__ int64_t first_w() const { return ((x0 + 1) * P - 1) / Nc; }
  __device__ int64_t last_w() const { return ((x1 + 1) * P - 1) / Nc; }
  __device__ bool owns(int64_t w) const {
    const int64_t s = start(w), e = start(w + 1);
    return s < e && e > x0 && s <= x1;
  }
};

template <typename Acc>
struct RowStats {
  Acc m, l;
};

// m and l of packed row r over the segments of its group (whole wave).
template <typename Acc>
__device__ RowStats<Acc> row_stats(const StepArgs& a, int64_t grp, int64_t nc, const StreamSegs& ss,
                                   int r, int lane) {
  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  Acc m = neg_inf;
  const int64_t k0 = a.seg_mode ? ss.first_w() : 0;
  const int64_t k1 = a.seg_mode ? ss.last_w() + 1 : nc;
  for (int64_t k = k0 + lane; k < k1; k += kWave) {
    if (a.seg_mode && !ss.owns(k)) continue;
    const int64_t seg = a.seg_mode ? k + grp : grp * a.nchunk_max + k;
    const Acc mk = static_cast<Acc>(a.ws_seg_ml[(seg * a.R + r) * 2]);
    m = mk > m ? mk : m;
  }
  m = wave_max(m);
  Acc l = 0;
  for (int64_t k = k0 + lane; k < k1; k += kWave) {
    if (a.seg_mode && !ss.owns(k)) continue;
    const int64_t seg = a.seg_mode ? k + grp : grp * a.nchunk_max + k;
    const Acc mk = static_cast<Acc>(a.ws_seg_ml[(seg * a.R + r) * 2]);
    if (mk != neg_inf) l += static_cast<Acc>(a.ws_seg_ml[(seg * a.R + r) * 2 + 1]) * acc_exp(mk - m);
  }
  l = wave_sum(l);
  return {m, l};
}

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(StepArgs a) {
  using E = Elem<T>;
  using Acc = typename E::Acc;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t ncw = ceil_div(a.M, a.CS);
  const int64_t k = blockIdx.x % ncw;
  const int64_t grp = blockIdx.x / ncw;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;
  const int64_t len = a.ws_rowinfo[b * 4 + 0];
  const int64_t n = a.ws_rowinfo[b * 4 + 1];
  const int32_t status = static_cast<int32_t>(a.ws_rowinfo[b * 4 + 2]);
  const int64_t nc = row_chunks(len, n, a.C);

  if (k == 0 && kvh == 0 && tid == 0) {
    a.lengths_out[b] = len + n;
    if (a.row_status) a.row_status[b] = status;
  }
  const int64_t e0 = k * a.CS;
  const int64_t e1 = e0 + a.CS < a.M ? e0 + a.CS : a.M;

  if (a.out_of_place && a.combine_copies_tail) {
    const int64_t cover = n > 0 ? len + n : 0;
    const int64_t j0 = e0 > cover ? e0 : cover;
    if (j0 < e1) {
      const int64_t kb = a.D * E::kBytes, vb = a.Dv * E::kBytes;
      const int64_t hk = grp * a.M;
      copy_bytes(static_cast<uint8_t*>(a.kc_out) + (hk + j0) * kb,
                 static_cast<const uint8_t*>(a.kc_in) + (hk + j0) * kb, (e1 - j0) * kb, tid,
                 kCombineThreads);
      copy_bytes(static_cast<uint8_t*>(a.vc_out) + (hk + j0) * vb,
                 static_cast<const uint8_t*>(a.vc_in) + (hk + j0) * vb, (e1 - j0) * vb, tid,
                 kCombineThreads);
    }
  }

  StreamSegs ss{0, a.P, 0, 0, grp};
  if (a.seg_mode && nc > 0) {
    ss.Nc = a.ws_hdr[0];
    ss.x0 = a.ws_rowinfo[b * 4 + 3] + kvh * nc;
    ss.x1 = ss.x0 + nc - 1;
  }
  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  T* att = static_cast<T*>(a.attention);
  T* ctx = static_cast<T*>(a.context);
  const double* chunk_ml = a.ws_chunk_ml + grp * a.nchunk_max * a.R * 2;

  for (int r = wave; r < a.R; r += kCombineThreads / kWave) {
    const int64_t g = r / a.Q, t = r % a.Q;
    const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
    const bool ctx_owner = (r % ncw) == k;
    T* arow = att + row * a.M;
    if (t >= n) {  // invalid row: zero attention and context
      for (int64_t j = e0 + lane; j < e1; j += kWave) arow[j] = E::zero();
      if (ctx_owner)
        for (int64_t dv = lane; dv < a.Dv; dv += kWave) ctx[row * a.Dv + dv] = E::zero();
      continue;
    }
    const int64_t lim = len + t + 1;  // slots [0, lim) are visible
    const int64_t v1 = e1 < lim ? e1 : lim;
    if (v1 > e0 || ctx_owner) {
      const RowStats<Acc> st = row_stats<Acc>(a, grp, nc, ss, r, lane);
      const Acc inv_l = Acc(1) / st.l;
      for (int64_t j = e0 + lane; j < v1; j += kWave) {
        const Acc mc = static_cast<Acc>(chunk_ml[((j / a.C) * a.R + r) * 2]);
        const Acc f = mc == neg_inf ? Acc(0) : acc_exp(mc - st.m) * inv_l;
        E::store(arow + j, E::load(arow + j) * f);
      }
      if (ctx_owner) {
        const int64_t k0 = a.seg_mode ? ss.first_w() : 0;
        const int64_t k1 = a.seg_mode ? ss.last_w() + 1 : nc;
        for (int64_t dv = lane; dv < a.Dv; dv += kWave) {
          Acc o = 0;
          for (int64_t s = k0; s < k1; s++) {
            if (a.seg_mode && !ss.owns(s)) continue;
            const int64_t seg = a.seg_mode ? s + grp : grp * a.nchunk_max + s;
            const Acc mk = static_cast<Acc>(a.ws_seg_ml[(seg * a.R + r) * 2]);
            if (mk == neg_inf) continue;
            o += static_cast<Acc>(a.ws_seg_o[(seg * a.R + r) * a.Dv + dv]) * acc_exp(mk - st.m);
          }
          E::store(ctx + row * a.Dv + dv, o * inv_l);
        }
      }
    }
    const int64_t z0 = v1 > e0 ? v1 : e0;
    for (int64_t j = z0 + lane; j < e1; j += kWave) arow[j] = E::zero();
  }
}

}  // namespace kvc
