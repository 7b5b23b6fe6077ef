// kvc_generic.h -- attend kernel for any head sizes (D, Dv) and any packed
// row count, in dense chunk mode (one workgroup per chunk and row tile).
// It is the path for shapes the vector decode kernel does not cover (odd
// head sizes, misaligned buffers, many packed rows) and for paged caches
// whose blocks are smaller than the other paths' chunks; it leaves the same
// chunk and segment results and shares the combine kernel.
//
// One workgroup handles one (batch row b, KV head h, row tile, chunk c):
//   1. cache writes for the chunk's slot range (row tile 0 only): the whole
//      range is copied when out of place, otherwise only the appended rows
//      are written ("Autoregressive KV-cache append and causal attention",
//      Required behavior: new rows at slot length + t, every other entry
//      kept bit for bit);
//   2. scores scale * dot(q, k) of its packed query rows against the slots
//      they may see (j <= length + t, the lower-right alignment of
//      KempnerForge PR 542, Summary); new rows are read from new_key /
//      new_value, so no workgroup depends on another's cache writes;
//   3. chunk statistics m_c = max s_j, l_c = sum exp(s_j - m_c), the
//      unnormalised context o_c = sum exp(s_j - m_c) v_j, and exp(s_j - m_c)
//      into the attention buffer; the chunk is its own segment.
#pragma once

#include "kvc_common.h"

namespace kvc {

constexpr int kGenericChunk = 256;     // slots per chunk
constexpr int kGenericRowsPerTile = 8; // packed query rows per workgroup
constexpr int kGenericThreads = 256;

// Copy nbytes from src to dst with the widest unit both addresses allow.
// The 16-byte path takes four pieces per thread per round, loaded before
// any of them is stored: the compiler cannot tell that src and dst do not
// overlap, and would otherwise wait for each load before its store.  The
// copied bytes are not used again by the step, so the accesses are
// non-temporal.
typedef unsigned int cu32x4 __attribute__((ext_vector_type(4)));
__device__ inline void copy_bytes(uint8_t* dst, const uint8_t* src, int64_t nbytes, int tid,
                                  int nthr) {
  if (nbytes <= 0) return;
  const uintptr_t al = reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) |
                       static_cast<uintptr_t>(nbytes);
  if ((al & 15u) == 0) {
    const int64_t n = nbytes / 16, step = nthr;
    uint4* d = reinterpret_cast<uint4*>(dst);
    const uint4* s = reinterpret_cast<const uint4*>(src);
    for (int64_t i = tid; i < n; i += 4 * step) {
      // past the end: the last piece again, not stored
      const int64_t k1 = i + step, k2 = i + 2 * step, k3 = i + 3 * step;
      const cu32x4* sv = reinterpret_cast<const cu32x4*>(s);
      cu32x4* dv = reinterpret_cast<cu32x4*>(d);
      const cu32x4 v0 = __builtin_nontemporal_load(sv + i);
      const cu32x4 v1 = __builtin_nontemporal_load(sv + (k1 < n ? k1 : n - 1));
      const cu32x4 v2 = __builtin_nontemporal_load(sv + (k2 < n ? k2 : n - 1));
      const cu32x4 v3 = __builtin_nontemporal_load(sv + (k3 < n ? k3 : n - 1));
      __builtin_nontemporal_store(v0, dv + i);
      if (k1 < n) __builtin_nontemporal_store(v1, dv + k1);
      if (k2 < n) __builtin_nontemporal_store(v2, dv + k2);
      if (k3 < n) __builtin_nontemporal_store(v3, dv + k3);
    }
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
  constexpr int C = kGenericChunk;
  __shared__ Acc sc[RT][C];
  __shared__ Acc row_m[RT], row_l[RT];
  __shared__ RowInfo info_sh;

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int64_t wg = blockIdx.x;
  const int64_t c = wg % a.nchunk_max;
  const int64_t rest = wg / a.nchunk_max;
  const int rt = static_cast<int>(rest % a.row_tiles);
  const int64_t grp = rest / a.row_tiles;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;

  if (wave == 0) {
    RowInfo ri = wave_row_info(a.lengths, a.mask, a.Q, a.M, b);
    if (lane == 0) info_sh = ri;
  }
  __syncthreads();
  const RowInfo ri = info_sh;
  if (c == 0 && kvh == 0 && rt == 0 && tid == 0) {
    a.ws_rowinfo[b * 4 + 0] = ri.len;
    a.ws_rowinfo[b * 4 + 1] = ri.n;
    a.ws_rowinfo[b * 4 + 2] = ri.status;
    a.ws_rowinfo[b * 4 + 3] = 0;
  }
  const int64_t len = ri.len, n = ri.n, new_len = len + n;
  const int64_t s0 = c * C;
  const int64_t s1 = s0 + C < a.M ? s0 + C : a.M;

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

  // slot j's key / value row of the updated caches: appended rows from the
  // new rows, kept ones from the cache (dense, or the paged pool; nullptr
  // for a table entry outside the pool, read as a zero row)
  const int64_t kb = a.D * E::kBytes, vb = a.Dv * E::kBytes;
  auto key_row = [&](int64_t j) -> const T* {
    if (j >= len) return nk_head + (j - len) * a.D;
    if (!a.paged) return k_head + j * a.D;
    return reinterpret_cast<const T*>(slot_row(a, a.kc_in, b, kvh, j, kb));
  };
  auto value_row = [&](int64_t j) -> const T* {
    if (j >= len) return nv_head + (j - len) * a.Dv;
    if (!a.paged) return v_head + j * a.Dv;
    return reinterpret_cast<const T*>(slot_row(a, a.vc_in, b, kvh, j, vb));
  };

  // 1. cache writes
  if (rt == 0 && !a.read_only && a.paged) {  // in place: the appended rows' blocks
    const int64_t m0 = s0 > len ? s0 : len, m1 = s1 < len + n ? s1 : len + n;
    for (int64_t j = m0; j < m1; j++) {
      uint8_t* kd = const_cast<uint8_t*>(slot_row(a, a.kc_out, b, kvh, j, kb));
      uint8_t* vd = const_cast<uint8_t*>(slot_row(a, a.vc_out, b, kvh, j, vb));
      if (kd)
        copy_bytes(kd, reinterpret_cast<const uint8_t*>(nk_head + (j - len) * a.D), kb, tid,
                   kGenericThreads);
      if (vd)
        copy_bytes(vd, reinterpret_cast<const uint8_t*>(nv_head + (j - len) * a.Dv), vb, tid,
                   kGenericThreads);
    }
  } else if (rt == 0 && !a.read_only) {
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
  if (rcount <= 0 || c >= row_chunks(len, n, C)) return;
  const int64_t act_end = s1 < new_len ? s1 : new_len;
  const int nact = static_cast<int>(act_end - s0);
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
      const T* kp = key_row(j);
      const T* qp = q + ((b * a.Hq + kvh * a.G + g) * a.Q + t) * a.D;
      Acc dot = 0;
      if (kp)
        for (int64_t d = 0; d < a.D; d++) dot += E::load(qp + d) * E::load(kp + d);
      val = scale * dot;
    }
    sc[r][idx % nact] = val;
  }
  __syncthreads();

  // 3. chunk statistics; p = exp(s - m_c) replaces the score in LDS
  T* att = static_cast<T*>(a.attention);
  for (int r = wave; r < rcount; r += kGenericThreads / kWave) {
    const int rg = r0 + r;
    const int64_t g = rg / a.Q, t = rg % a.Q;
    Acc m = neg_inf;
    for (int i = lane; i < nact; i += kWave) m = sc[r][i] > m ? sc[r][i] : m;
    m = wave_max(m);
    Acc l = 0;
    T* arow = att + ((b * a.Hq + kvh * a.G + g) * a.Q + t) * a.M + s0;
    for (int i = lane; i < nact; i += kWave) {
      const Acc p = (m == neg_inf || sc[r][i] == neg_inf) ? Acc(0) : acc_exp(sc[r][i] - m);
      sc[r][i] = p;
      l += p;
      if (t < n && !a.read_only) E::store(arow + i, p);
    }
    l = wave_sum(l);
    if (lane == 0) {
      row_m[r] = m;
      row_l[r] = l;
      if (t < n) {
        double* cm = a.ws_chunk_ml + ((grp * a.nchunk_max + c) * a.R + rg) * 2;
        cm[0] = static_cast<double>(m);
        cm[1] = static_cast<double>(l);
      }
    }
  }
  __syncthreads();

  // segment = this chunk: statistics and o_c = sum_j p_j v_j
  const int64_t seg = grp * a.nchunk_max + c;
  for (int idx = tid; idx < rcount * a.Dv; idx += kGenericThreads) {
    const int r = static_cast<int>(idx / a.Dv);
    const int64_t dv = idx % a.Dv;
    const int rg = r0 + r;
    const int64_t t = rg % a.Q;
    if (t >= n) continue;
    Acc o = 0;
    for (int i = 0; i < nact; i++) {
      const int64_t j = s0 + i;
      const T* vp = value_row(j);
      if (vp) o += sc[r][i] * E::load(vp + dv);
    }
    a.ws_seg_o[(seg * a.R + rg) * a.Dv + dv] = static_cast<float>(o);
  }
  for (int r = tid; r < rcount; r += kGenericThreads) {
    double* ml = a.ws_seg_ml + (seg * a.R + r0 + r) * 2;
    ml[0] = static_cast<double>(row_m[r]);
    ml[1] = static_cast<double>(row_l[r]);
  }
}

}  // namespace kvc
