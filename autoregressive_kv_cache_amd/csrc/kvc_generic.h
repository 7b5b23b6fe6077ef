// kvc_generic.h -- split-K attention kernel for any head sizes (D, Dv) and
// any packed row count.  It is the path for shapes the vector decode and
// MFMA chunk kernels do not cover (odd head sizes, tiny problems); those
// kernels follow the same split protocol and share the combine kernel.
//
// One workgroup handles one (batch row b, KV head h, row tile, split s):
//   1. cache writes for its slot range (row tile 0 only): the whole range is
//      copied when out of place, otherwise only the appended rows are
//      written ("Autoregressive KV-cache append and causal attention",
//      Required behavior: new rows at slot length + t, every other entry
//      kept bit for bit);
//   2. scores scale * dot(q, k) of its packed query rows against the slots
//      they may see (j <= length + t, the lower-right alignment of
//      KempnerForge PR 542, Summary); new rows are read from new_key /
//      new_value, so no workgroup depends on another's cache writes;
//   3. split softmax statistics m_s = max s_j, l_s = sum exp(s_j - m_s)
//      and the unnormalised context o_s = sum exp(s_j - m_s) v_j;
//   4. when the batch row has a single active split the outputs are final
//      (attention = p / l, context = o / l); otherwise exp(s_j - m_s) goes to
//      the attention buffer and (m_s, l_s, o_s) to the workspace for the
//      combine kernel.
#pragma once

#include "kvc_common.h"

namespace kvc {

constexpr int kGenericSplit = 256;     // slots per split
constexpr int kGenericRowsPerTile = 8; // packed query rows per workgroup
constexpr int kGenericThreads = 256;

// Copy nbytes from src to dst with the widest unit both addresses allow.
__device__ inline void copy_bytes(uint8_t* dst, const uint8_t* src, int64_t nbytes, int tid,
                                  int nthr) {
  if (nbytes <= 0) return;
  const uintptr_t al = reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) |
                       static_cast<uintptr_t>(nbytes);
  if ((al & 15u) == 0) {
    const int64_t n = nbytes / 16;
    uint4* d = reinterpret_cast<uint4*>(dst);
    const uint4* s = reinterpret_cast<const uint4*>(src);
    for (int64_t i = tid; i < n; i += nthr) d[i] = s[i];
  } else {
    const int64_t n = nbytes / 2;
    uint16_t* d = reinterpret_cast<uint16_t*>(dst);
    const uint16_t* s = reinterpret_cast<const uint16_t*>(src);
    for (int64_t i = tid; i < n; i += nthr) d[i] = s[i];
  }
}

// Cache writes for slots [j0, j1) of one (b, h) head of one cache tensor
// with rows of `row_bytes`.  Out of place: every slot is written (from the
// input cache, or from the new rows for slots len .. len+n-1).  In place:
// only the new rows.
__device__ inline void write_cache_slots(uint8_t* dst_head, const uint8_t* src_head,
                                         const uint8_t* new_head, int64_t row_bytes, int64_t j0,
                                         int64_t j1, int64_t len, int64_t n, bool out_of_place,
                                         int tid, int nthr) {
  const int64_t a0 = j0, a1 = j1 < len ? j1 : len;            // old prefix part
  const int64_t m0 = j0 > len ? j0 : len;                      // appended part
  const int64_t m1 = j1 < len + n ? j1 : len + n;
  const int64_t t0 = j0 > len + n ? j0 : len + n, t1 = j1;    // tail part
  if (out_of_place) {
    if (n == 0) {
      copy_bytes(dst_head + j0 * row_bytes, src_head + j0 * row_bytes, (j1 - j0) * row_bytes, tid,
                 nthr);
      return;
    }
    copy_bytes(dst_head + a0 * row_bytes, src_head + a0 * row_bytes, (a1 - a0) * row_bytes, tid,
               nthr);
    copy_bytes(dst_head + t0 * row_bytes, src_head + t0 * row_bytes, (t1 - t0) * row_bytes, tid,
               nthr);
  }
  if (n > 0 && m1 > m0)
    copy_bytes(dst_head + m0 * row_bytes, new_head + (m0 - len) * row_bytes,
               (m1 - m0) * row_bytes, tid, nthr);
}

template <typename T>
__global__ __launch_bounds__(kGenericThreads) void attend_generic_kernel(StepArgs a) {
  using E = Elem<T>;
  using Acc = typename E::Acc;
  constexpr int RT = kGenericRowsPerTile;
  constexpr int S = kGenericSplit;
  __shared__ Acc sc[RT][S];
  __shared__ Acc row_m[RT], row_l[RT];
  __shared__ RowInfo info_sh;

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t wg = blockIdx.x;
  const int64_t s = wg % a.nsplit;
  const int64_t rest = wg / a.nsplit;
  const int rt = static_cast<int>(rest % a.row_tiles);
  const int64_t grp = rest / a.row_tiles;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;

  if (wave == 0) {
    RowInfo ri = wave_row_info(a.lengths, a.mask, a.Q, a.M, b);
    if (lane == 0) info_sh = ri;
  }
  __syncthreads();
  const RowInfo ri = info_sh;
  if (s == 0 && kvh == 0 && rt == 0 && tid == 0) {
    a.ws_rowinfo[b * 4 + 0] = ri.len;
    a.ws_rowinfo[b * 4 + 1] = ri.n;
    a.ws_rowinfo[b * 4 + 2] = ri.status;
  }
  const int64_t len = ri.len, n = ri.n, new_len = len + n;
  const int64_t s0 = s * S;
  const int64_t s1 = s0 + S < a.M ? s0 + S : a.M;

  const T* q = static_cast<const T*>(a.query);
  const T* nk = static_cast<const T*>(a.new_key);
  const T* nv = static_cast<const T*>(a.new_value);
  const T* kin = static_cast<const T*>(a.kc_in);
  const T* vin = static_cast<const T*>(a.vc_in);
  const int64_t head = b * a.Hk + kvh;
  const T* k_head = kin + head * a.M * a.D;
  const T* v_head = vin + head * a.M * a.Dv;
  const T* nk_head = nk + head * a.Q * a.D;
  const T* nv_head = nv + head * a.Q * a.Dv;

  // 1. cache writes
  if (rt == 0) {
    const int64_t kb = a.D * E::kBytes, vb = a.Dv * E::kBytes;
    write_cache_slots(static_cast<uint8_t*>(a.kc_out) + head * a.M * kb,
                      reinterpret_cast<const uint8_t*>(k_head),
                      reinterpret_cast<const uint8_t*>(nk_head), kb, s0, s1, len, n,
                      a.out_of_place != 0, tid, kGenericThreads);
    write_cache_slots(static_cast<uint8_t*>(a.vc_out) + head * a.M * vb,
                      reinterpret_cast<const uint8_t*>(v_head),
                      reinterpret_cast<const uint8_t*>(nv_head), vb, s0, s1, len, n,
                      a.out_of_place != 0, tid, kGenericThreads);
  }

  const int r0 = rt * RT;
  const int rcount = a.R - r0 < RT ? a.R - r0 : RT;
  if (rcount <= 0) return;
  const int64_t nsa = active_splits(len, n, S);
  const int64_t act_end = (n > 0) ? (s1 < new_len ? s1 : new_len) : s0;
  const int nact = act_end > s0 ? static_cast<int>(act_end - s0) : 0;
  const Acc scale = static_cast<Acc>(a.scale);
  const Acc neg_inf = -static_cast<Acc>(INFINITY);

  // 2. scores
  for (int idx = tid; idx < rcount * nact; idx += kGenericThreads) {
    const int r = idx / nact;
    const int64_t j = s0 + idx % nact;
    const int rg = r0 + r;
    const int64_t g = rg / a.Q, t = rg % a.Q;
    Acc val = neg_inf;
    if (t < n && j <= len + t) {
      const T* kp = j < len ? k_head + j * a.D : nk_head + (j - len) * a.D;
      const T* qp = q + ((b * a.Hq + kvh * a.G + g) * a.Q + t) * a.D;
      Acc dot = 0;
      for (int64_t d = 0; d < a.D; d++) dot += E::load(qp + d) * E::load(kp + d);
      val = scale * dot;
    }
    sc[r][idx % nact] = val;
  }
  __syncthreads();

  // 3. split statistics; p = exp(s - m_s) replaces the score in LDS
  for (int r = wave; r < rcount; r += kGenericThreads / kWave) {
    Acc m = neg_inf;
    for (int i = lane; i < nact; i += kWave) m = sc[r][i] > m ? sc[r][i] : m;
    m = wave_max(m);
    Acc l = 0;
    for (int i = lane; i < nact; i += kWave) {
      const Acc p = (m == neg_inf || sc[r][i] == neg_inf) ? Acc(0) : acc_exp(sc[r][i] - m);
      sc[r][i] = p;
      l += p;
    }
    l = wave_sum(l);
    if (lane == 0) {
      row_m[r] = m;
      row_l[r] = l;
    }
  }
  __syncthreads();

  const bool single = (nsa == 1);
  T* att = static_cast<T*>(a.attention);
  // attention rows of this tile over [s0, s1)
  for (int r = 0; r < rcount; r++) {
    const int rg = r0 + r;
    const int64_t g = rg / a.Q, t = rg % a.Q;
    T* arow = att + ((b * a.Hq + kvh * a.G + g) * a.Q + t) * a.M;
    const Acc inv_l = (single && row_l[r] > 0) ? Acc(1) / row_l[r] : Acc(1);
    for (int64_t j = s0 + tid; j < s1; j += kGenericThreads) {
      const int i = static_cast<int>(j - s0);
      const Acc p = i < nact ? sc[r][i] : Acc(0);
      E::store(arow + j, single ? p * inv_l : p);
    }
  }

  // context pieces: o[r][dv] = sum_j p_j v_j over this split
  T* ctx = static_cast<T*>(a.context);
  const bool write_ctx = (s == 0 && nsa <= 1);
  const bool write_part = (!single && s < nsa);
  for (int idx = tid; idx < rcount * a.Dv; idx += kGenericThreads) {
    const int r = static_cast<int>(idx / a.Dv);
    const int64_t dv = idx % a.Dv;
    const int rg = r0 + r;
    const int64_t g = rg / a.Q, t = rg % a.Q;
    Acc o = 0;
    if (t < n) {
      for (int i = 0; i < nact; i++) {
        const int64_t j = s0 + i;
        const T* vp = j < len ? v_head + j * a.Dv : nv_head + (j - len) * a.Dv;
        o += sc[r][i] * E::load(vp + dv);
      }
    }
    if (write_ctx) {
      const Acc val = (t < n && row_l[r] > 0) ? o / row_l[r] : Acc(0);
      E::store(ctx + ((b * a.Hq + kvh * a.G + g) * a.Q + t) * a.Dv + dv, val);
    }
    if (write_part) a.ws_o[((grp * a.nsplit + s) * a.R + rg) * a.Dv + dv] = static_cast<float>(o);
  }
  if (write_part) {
    for (int r = tid; r < rcount; r += kGenericThreads) {
      double* ml = a.ws_ml + ((grp * a.nsplit + s) * a.R + r0 + r) * 2;
      ml[0] = static_cast<double>(row_m[r]);
      ml[1] = static_cast<double>(row_l[r]);
    }
  }
}

}  // namespace kvc
