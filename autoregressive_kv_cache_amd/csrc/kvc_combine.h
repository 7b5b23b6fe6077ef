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

constexpr int kCombineWaves = 4;
constexpr int kCombineThreads = kCombineWaves * kWave;

// The segments of one group: ids first + s for s in [0, count).  Stream
// mode: the workers owning chunks [x0, x1] of the flattened list are
// consecutive, segment id = worker + group.  Dense mode: one per chunk.
struct SegRange {
  int64_t first, count;
};

// first_chunk: the row's first chunk in the flattened list (row record
// entry 3); Nc, Pe: header entries 0 and 1 (all loaded by the caller with
// the row record, so that no load waits on another).
__device__ inline SegRange group_segments(const StepArgs& a, int64_t grp, int64_t kvh, int64_t nc,
                                          int64_t first_chunk, int64_t Nc, int64_t Pe) {
  if (nc <= 0) return {0, 0};
  if (!a.seg_mode) return {grp * a.nchunk_max, nc};
  const int64_t x0 = first_chunk + kvh * nc, x1 = x0 + nc - 1;
  const int32_t lead = effective_lead(Nc, Pe, a.lead);
  const int64_t w0 = worker_owner(x0, Nc, Pe, lead), w1 = worker_owner(x1, Nc, Pe, lead);
  return {w0 + grp, w1 - w0 + 1};
}

// Eight consecutive elements of T (16 bytes of bf16, 32 of fp32).
template <typename T>
struct Vec8;
// The combine reads each exponential once and writes each attention entry
// once: both go through non-temporal accesses, which do not keep the lines
// in the caches (the next step's K/V rows then find them emptier).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
template <>
struct Vec8<bf16> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16* p) {
    const nt_u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
    v = make_uint4(w.x, w.y, w.z, w.w);
  }
  __device__ __forceinline__ void store(bf16* p) const {
    const nt_u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<nt_u32x4*>(p));
  }
  __device__ __forceinline__ void scale_by(float f) {
    uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t lo = f32_to_bf16(__uint_as_float(w[k] << 16) * f);
      const uint32_t hi = f32_to_bf16(__uint_as_float(w[k] & 0xffff0000u) * f);
      w[k] = lo | (hi << 16);
    }
  }
  // elements [0, k) scaled by f_lo, the others by f_hi
  __device__ __forceinline__ void scale_split(float f_lo, float f_hi, int k) {
    uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const uint32_t lo = f32_to_bf16(__uint_as_float(w[e] << 16) * (2 * e < k ? f_lo : f_hi));
      const uint32_t hi =
          f32_to_bf16(__uint_as_float(w[e] & 0xffff0000u) * (2 * e + 1 < k ? f_lo : f_hi));
      w[e] = lo | (hi << 16);
    }
  }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  // keep elements [0, cnt), zero the others (no indexed access: the vector
  // stays in registers)
  __device__ __forceinline__ void keep_first(int cnt) {
    v.x &= (cnt > 0 ? 0xffffu : 0u) | (cnt > 1 ? 0xffff0000u : 0u);
    v.y &= (cnt > 2 ? 0xffffu : 0u) | (cnt > 3 ? 0xffff0000u : 0u);
    v.z &= (cnt > 4 ? 0xffffu : 0u) | (cnt > 5 ? 0xffff0000u : 0u);
    v.w &= (cnt > 6 ? 0xffffu : 0u) | (cnt > 7 ? 0xffff0000u : 0u);
  }
};
template <>
struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    const nt_f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
    const nt_f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p) + 1);
    a = make_float4(x.x, x.y, x.z, x.w);
    b = make_float4(y.x, y.y, y.z, y.w);
  }
  __device__ __forceinline__ void store(float* p) const {
    const nt_f32x4 x = {a.x, a.y, a.z, a.w}, y = {b.x, b.y, b.z, b.w};
    __builtin_nontemporal_store(x, reinterpret_cast<nt_f32x4*>(p));
    __builtin_nontemporal_store(y, reinterpret_cast<nt_f32x4*>(p) + 1);
  }
  __device__ __forceinline__ void scale_by(double f) {
    a.x = static_cast<float>(a.x * f); a.y = static_cast<float>(a.y * f);
    a.z = static_cast<float>(a.z * f); a.w = static_cast<float>(a.w * f);
    b.x = static_cast<float>(b.x * f); b.y = static_cast<float>(b.y * f);
    b.z = static_cast<float>(b.z * f); b.w = static_cast<float>(b.w * f);
  }
  __device__ __forceinline__ void scale_split(double f_lo, double f_hi, int k) {
    a.x = static_cast<float>(a.x * (k > 0 ? f_lo : f_hi));
    a.y = static_cast<float>(a.y * (k > 1 ? f_lo : f_hi));
    a.z = static_cast<float>(a.z * (k > 2 ? f_lo : f_hi));
    a.w = static_cast<float>(a.w * (k > 3 ? f_lo : f_hi));
    b.x = static_cast<float>(b.x * (k > 4 ? f_lo : f_hi));
    b.y = static_cast<float>(b.y * (k > 5 ? f_lo : f_hi));
    b.z = static_cast<float>(b.z * (k > 6 ? f_lo : f_hi));
    b.w = static_cast<float>(b.w * (k > 7 ? f_lo : f_hi));
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void keep_first(int cnt) {
    a.x = cnt > 0 ? a.x : 0.f; a.y = cnt > 1 ? a.y : 0.f;
    a.z = cnt > 2 ? a.z : 0.f; a.w = cnt > 3 ? a.w : 0.f;
    b.x = cnt > 4 ? b.x : 0.f; b.y = cnt > 5 ? b.y : 0.f;
    b.z = cnt > 6 ? b.z : 0.f; b.w = cnt > 7 ? b.w : 0.f;
  }
};

constexpr int kCombineVecPerLane = 8;  // 8-element vectors per lane and pass

// Workgroup = kCombineWaves waves; wave w owns packed row rb * kCombineWaves + w
// of its group.  Workgroups k < ceil(M / CS) rescale the slot range
// [k * CS, (k + 1) * CS) of their rows; workgroup k = ceil(M / CS) merges
// their contexts, in parallel with the rescaling.  Every wave works alone:
// the attention vectors, the chunk statistics, the segment statistics and
// (context role) the first segment partials it needs are all requested
// before any of them is used.
template <typename T>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(StepArgs a) {
  using E = Elem<T>;
  using Acc = typename E::Acc;
  constexpr int VPL = kCombineVecPerLane;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int64_t ncw = ceil_div(a.M, a.CS);
  const int64_t nrb = a.R > 0 ? ceil_div(a.R, kCombineWaves) : 1;
  // read-only (re-attention): only the context is wanted -- the grid holds
  // the context role of each group alone, and no attention row is written
  const int64_t rb = blockIdx.x % nrb;
  const int64_t k = a.read_only ? ncw : (blockIdx.x / nrb) % (ncw + 1);
  const int64_t grp = a.read_only ? blockIdx.x / nrb : blockIdx.x / nrb / (ncw + 1);
  const bool ctx_role = k == ncw;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;
  // the row record and the stream header in one round of loads
  const int64_t len = a.ws_rowinfo[b * 4 + 0];
  const int64_t n = a.ws_rowinfo[b * 4 + 1];
  const int32_t status = static_cast<int32_t>(a.ws_rowinfo[b * 4 + 2]);
  const int64_t first_chunk = a.ws_rowinfo[b * 4 + 3];
  const int64_t hdr_nc = a.ws_hdr[0], hdr_pe = a.ws_hdr[1];
  const int64_t nc = a.seg_mode ? stream_chunks(len, n, a.C) : row_chunks(len, n, a.C);
  // chunk holding slot j (stream mode: the appended rows are a chunk of
  // their own, so an 8-slot vector may straddle two chunks at slot len)
  const int64_t len_chunks = (len + a.C - 1) >> a.C_log2;  // cached chunks (stream mode)
  auto chunk_of = [&](int64_t j) {
    return a.seg_mode && j >= len ? len_chunks : j >> a.C_log2;
  };

  if ((a.read_only ? ctx_role : k == 0) && kvh == 0 && rb == 0 && tid == 0) {
    a.lengths_out[b] = len + n;
    if (a.row_status) a.row_status[b] = status;
  }
  const int64_t e0 = ctx_role ? a.M : k * a.CS;
  const int64_t e1 = e0 + a.CS < a.M ? e0 + a.CS : a.M;

  if (ctx_role && rb == 0 && a.seg_mode && !a.out_of_place && !a.read_only && n > 0) {
    // in place, stream path: the appended rows go to their cache slots
    // (the attend kernel read them from new_key / new_value)
    const int64_t kb = a.D * E::kBytes, vb = a.Dv * E::kBytes;
    const uint8_t* nk = static_cast<const uint8_t*>(a.new_key) + grp * a.Q * kb;
    const uint8_t* nv = static_cast<const uint8_t*>(a.new_value) + grp * a.Q * vb;
    if (!a.paged) {
      copy_bytes(static_cast<uint8_t*>(a.kc_out) + (grp * a.M + len) * kb, nk, n * kb, tid,
                 kCombineThreads);
      copy_bytes(static_cast<uint8_t*>(a.vc_out) + (grp * a.M + len) * vb, nv, n * vb, tid,
                 kCombineThreads);
    } else {
      // one row at a time: consecutive slots may lie in different blocks
      for (int64_t t = 0; t < n; t++) {
        uint8_t* kd = const_cast<uint8_t*>(slot_row(a, a.kc_out, b, kvh, len + t, kb));
        uint8_t* vd = const_cast<uint8_t*>(slot_row(a, a.vc_out, b, kvh, len + t, vb));
        if (kd) copy_bytes(kd, nk + t * kb, kb, tid, kCombineThreads);
        if (vd) copy_bytes(vd, nv + t * vb, vb, tid, kCombineThreads);
      }
    }
  }
  if (rb == 0 && a.out_of_place && a.combine_copies_tail) {
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

  const int64_t r = rb * kCombineWaves + wave;
  if (r >= a.R) return;
  const int64_t g = r / a.Q, t = r % a.Q;
  const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
  const int64_t lim = t < n ? len + t + 1 : 0;  // visible slots [0, lim)
  const bool owns_ctx = ctx_role;
  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  T* arow = static_cast<T*>(a.attention) + row * a.M;
  T* ctx = static_cast<T*>(a.context) + row * a.Dv;
  const double* chunk_ml = a.ws_chunk_ml + grp * a.nchunk_max * a.R * 2;
  const SegRange sr = group_segments(a, grp, kvh, nc, first_chunk, hdr_nc, hdr_pe);
  // 8-element vectors need 16-byte aligned rows and ranges
  const bool vec = (reinterpret_cast<uintptr_t>(a.attention) % 16 == 0) && (a.M % 8 == 0) &&
                   (e0 % 8 == 0) && (e1 % 8 == 0);

  // ---- first pass of the range: its loads go out before the statistics ----
  const int64_t nvec = (e1 - e0) / 8;
  Vec8<T> x[VPL];
  Acc mc[VPL], mc_hi[VPL];
  int split[VPL];  // elements of the vector in the chunk of its first slot
  // The chunk maxima are converted as they are loaded: keeping them as
  // loaded (fp64) to defer that wait costs 8 more registers per lane, which
  // drops the bf16 kernel from 5 to 4 waves per SIMD and is slower.
  auto load_vec = [&](int v, int64_t vi) {
    const int64_t base = e0 + vi * 8;
    const bool live = vi < nvec && base < lim;
    // the vector's last slot may lie in the next chunk (stream mode, at len)
    const int64_t last = base + 7 < lim ? base + 7 : lim - 1;
    x[v].zero();
    if (live) x[v].load(arow + base);
    mc[v] = live ? static_cast<Acc>(chunk_ml[(chunk_of(base) * a.R + r) * 2]) : neg_inf;
    mc_hi[v] = live ? static_cast<Acc>(chunk_ml[(chunk_of(last) * a.R + r) * 2]) : neg_inf;
    split[v] = a.seg_mode && base < len && base + 8 > len ? static_cast<int>(len - base) : 8;
  };
  if (vec) {
#pragma unroll
    for (int v = 0; v < VPL; v++) load_vec(v, v * kWave + lane);
  }

  // segment statistics of the first kWave segments (lane s holds segment s)
  // and, for the wave that writes the row's context, the first batch of
  // segment partials: all requested before anything waits on them
  constexpr int SB = 16;
  const bool do_ctx = owns_ctx && t < n && sr.count > 0;
  double seg_m0 = -INFINITY, seg_l0 = 0;
  if (t < n && lane < sr.count) {
    const double* ml = a.ws_seg_ml + ((sr.first + lane) * a.R + r) * 2;
    seg_m0 = ml[0];
    seg_l0 = ml[1];
  }
  float cv[SB][2];
  auto load_batch = [&](int64_t s1, int64_t dv0) {
#pragma unroll
    for (int s = 0; s < SB; s++) {
      const float* op = a.ws_seg_o + ((sr.first + s1 + s) * a.R + r) * a.Dv;
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const int64_t dv = dv0 + q * kWave + lane;
        cv[s][q] = (s1 + s < sr.count && dv < a.Dv) ? op[dv] : 0.0f;
      }
    }
  };
  if (do_ctx) load_batch(0, 0);

  // ---- m and 1/l of the row over its segments (online merge) ----
  Acc m = neg_inf, l = 0;
  if (t < n) {
    auto merge = [&](Acc ms, Acc ls) {
      if (ms != neg_inf) {
        const Acc mn = ms > m ? ms : m;
        l = (m == neg_inf ? Acc(0) : l * acc_exp(m - mn)) + ls * acc_exp(ms - mn);
        m = mn;
      }
    };
    merge(static_cast<Acc>(seg_m0), static_cast<Acc>(seg_l0));
    for (int64_t s = kWave + lane; s < sr.count; s += kWave) {
      const double* ml = a.ws_seg_ml + ((sr.first + s) * a.R + r) * 2;
      merge(static_cast<Acc>(ml[0]), static_cast<Acc>(ml[1]));
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const Acc mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
      const Acc mn = mo > m ? mo : m;
      if (mn != neg_inf)
        l = (m == neg_inf ? Acc(0) : l * acc_exp(m - mn)) +
            (mo == neg_inf ? Acc(0) : lo * acc_exp(mo - mn));
      m = mn;
    }
  }
  if (t < n && a.sinks) {  // the head's sink: one more logit, no value row
    const Acc sk = static_cast<Acc>(a.sinks[kvh * a.G + g]);
    const Acc mn = sk > m ? sk : m;
    l = (m == neg_inf ? Acc(0) : l * acc_exp(m - mn)) + acc_exp(sk - mn);
    m = mn;
  }
  const Acc inv_l = l > 0 ? Acc(1) / l : Acc(0);
  auto factor = [&](Acc m_c) -> Acc { return m_c == neg_inf ? Acc(0) : acc_exp(m_c - m) * inv_l; };

  // ---- rescale the visible slots, zero the rest ----
  if (vec) {
    for (int64_t v0 = 0; v0 < nvec; v0 += VPL * kWave) {
      if (v0 > 0) {  // later passes (ranges longer than VPL * 512 slots)
#pragma unroll
        for (int v = 0; v < VPL; v++) load_vec(v, v0 + v * kWave + lane);
      }
#pragma unroll
      for (int v = 0; v < VPL; v++) {
        const int64_t base = e0 + (v0 + v * kWave + lane) * 8;
        if (v0 + v * kWave + lane < nvec) {
          if (base < lim) {
            x[v].scale_split(factor(mc[v]), factor(mc_hi[v]), split[v]);
            if (base + 8 > lim) x[v].keep_first(static_cast<int>(lim - base));
          }
          x[v].store(arow + base);
        }
      }
    }
  } else {
    for (int64_t j = e0 + lane; j < e1; j += kWave) {
      if (j < lim)
        E::store(arow + j, E::load(arow + j) *
                               factor(static_cast<Acc>(chunk_ml[(chunk_of(j) * a.R + r) * 2])));
      else
        arow[j] = E::zero();
    }
  }

  // ---- context of the rows this range owns ----
  if (!owns_ctx) return;
  if (!do_ctx) {
    for (int64_t dv = lane; dv < a.Dv; dv += kWave) ctx[dv] = E::zero();
    return;
  }
  // lanes own dims dv0 + q * 64 + lane, q < 2
  for (int64_t dv0 = 0; dv0 < a.Dv; dv0 += 2 * kWave) {
    Acc o[2] = {0, 0};
    for (int64_t s0 = 0; s0 < sr.count; s0 += kWave) {
      // weight of segment s0 + lane; broadcast one segment at a time
      Acc w = 0;
      if (s0 == 0) {
        w = factor(static_cast<Acc>(seg_m0));
      } else if (s0 + lane < sr.count) {
        w = factor(static_cast<Acc>(a.ws_seg_ml[((sr.first + s0 + lane) * a.R + r) * 2]));
      }
      const int64_t ns = sr.count - s0 < kWave ? sr.count - s0 : kWave;
      for (int64_t s1 = 0; s1 < ns; s1 += SB) {
        if (dv0 > 0 || s0 > 0 || s1 > 0) load_batch(s0 + s1, dv0);
#pragma unroll
        for (int s = 0; s < SB; s++) {
          const Acc ws = __shfl(w, static_cast<int>(s1 + s));  // 0 past the last segment
#pragma unroll
          for (int q = 0; q < 2; q++) o[q] += ws * static_cast<Acc>(cv[s][q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int64_t dv = dv0 + q * kWave + lane;
      if (dv < a.Dv) E::store(ctx + dv, o[q]);
    }
  }
}

}  // namespace kvc
