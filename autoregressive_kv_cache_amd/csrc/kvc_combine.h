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

// The segments of one group: ids first + s for s in [0, count).  Stream
// mode: the workers owning chunks [x0, x1] of the flattened list are
// consecutive, segment id = worker + group.  Dense mode: one per chunk.
struct SegRange {
  int64_t first, count;
};

__device__ inline SegRange group_segments(const StepArgs& a, int64_t grp, int64_t b, int64_t kvh,
                                          int64_t nc) {
  if (nc <= 0) return {0, 0};
  if (!a.seg_mode) return {grp * a.nchunk_max, nc};
  const int64_t Nc = a.ws_hdr[0], Pe = a.ws_hdr[1];
  const int64_t x0 = a.ws_rowinfo[b * 4 + 3] + kvh * nc, x1 = x0 + nc - 1;
  // owner(x) = the worker w with floor(w*Nc/Pe) <= x < floor((w+1)*Nc/Pe)
  const int64_t w0 = ((x0 + 1) * Pe - 1) / Nc, w1 = ((x1 + 1) * Pe - 1) / Nc;
  return {w0 + grp, w1 - w0 + 1};
}

template <typename Acc>
struct RowStats {
  Acc m, l;
};

// m and l of packed row r over the segments of its group (whole wave).
template <typename Acc>
__device__ RowStats<Acc> row_stats(const StepArgs& a, const SegRange& sr, int r, int lane) {
  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  Acc m = neg_inf;
  for (int64_t s = lane; s < sr.count; s += kWave) {
    const Acc mk = static_cast<Acc>(a.ws_seg_ml[((sr.first + s) * a.R + r) * 2]);
    m = mk > m ? mk : m;
  }
  m = wave_max(m);
  Acc l = 0;
  for (int64_t s = lane; s < sr.count; s += kWave) {
    const double* ml = a.ws_seg_ml + ((sr.first + s) * a.R + r) * 2;
    const Acc mk = static_cast<Acc>(ml[0]);
    if (mk != neg_inf) l += static_cast<Acc>(ml[1]) * acc_exp(mk - m);
  }
  l = wave_sum(l);
  return {m, l};
}

// Eight consecutive elements of T (16 bytes of bf16, 32 of fp32).
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void store(bf16* p) const { *reinterpret_cast<uint4*>(p) = v; }
  __device__ __forceinline__ void scale_by(float f) {
    uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t lo = f32_to_bf16(__uint_as_float(w[k] << 16) * f);
      const uint32_t hi = f32_to_bf16(__uint_as_float(w[k] & 0xffff0000u) * f);
      w[k] = lo | (hi << 16);
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
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = a;
    reinterpret_cast<float4*>(p)[1] = b;
  }
  __device__ __forceinline__ void scale_by(double f) {
    a.x = static_cast<float>(a.x * f); a.y = static_cast<float>(a.y * f);
    a.z = static_cast<float>(a.z * f); a.w = static_cast<float>(a.w * f);
    b.x = static_cast<float>(b.x * f); b.y = static_cast<float>(b.y * f);
    b.z = static_cast<float>(b.z * f); b.w = static_cast<float>(b.w * f);
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void keep_first(int cnt) {
    a.x = cnt > 0 ? a.x : 0.f; a.y = cnt > 1 ? a.y : 0.f;
    a.z = cnt > 2 ? a.z : 0.f; a.w = cnt > 3 ? a.w : 0.f;
    b.x = cnt > 4 ? b.x : 0.f; b.y = cnt > 5 ? b.y : 0.f;
    b.z = cnt > 6 ? b.z : 0.f; b.w = cnt > 7 ? b.w : 0.f;
  }
};

constexpr int kCombineRowBlock = 8;   // packed rows per pass
constexpr int kCombineMaxChunks = 64; // chunks per combine range (CS / C)

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(StepArgs a) {
  using E = Elem<T>;
  using Acc = typename E::Acc;
  constexpr int RB = kCombineRowBlock;
  __shared__ Acc row_m[RB], row_inv_l[RB];
  __shared__ Acc fac[RB][kCombineMaxChunks];
  __shared__ Acc seg_w[kCombineThreads];
  __shared__ Acc ctx_red[kCombineThreads];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
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
  const int nchunks = static_cast<int>(ceil_div(e1 - e0, a.C));  // chunks in this range
  const int64_t c0 = e0 / a.C;                                   // first chunk index

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

  const SegRange sr = group_segments(a, grp, b, kvh, nc);
  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  T* att = static_cast<T*>(a.attention);
  T* ctx = static_cast<T*>(a.context);
  const double* chunk_ml = a.ws_chunk_ml + grp * a.nchunk_max * a.R * 2;
  // 8-element vectors need 16-byte aligned rows and ranges
  const bool vec = (reinterpret_cast<uintptr_t>(att) % 16 == 0) && (a.M % 8 == 0) &&
                   (e0 % 8 == 0);

  for (int rb = 0; rb < a.R; rb += RB) {
    const int nrows = a.R - rb < RB ? static_cast<int>(a.R - rb) : RB;
    // 1. row statistics (m, 1/l) of the block's valid rows
    for (int i = wave; i < nrows; i += kCombineThreads / kWave) {
      const int r = rb + i;
      const int64_t t = r % a.Q;
      const bool need = t < n && (len + t + 1 > e0 || (r % ncw) == k);
      if (need) {
        const RowStats<Acc> st = row_stats<Acc>(a, sr, r, lane);
        if (lane == 0) {
          row_m[i] = st.m;
          row_inv_l[i] = Acc(1) / st.l;
        }
      }
    }
    __syncthreads();
    // 2. one factor exp(m_c - m) / l per (row, chunk) of the range
    for (int idx = tid; idx < nrows * nchunks; idx += kCombineThreads) {
      const int i = idx / nchunks, cc = idx % nchunks;
      const int r = rb + i;
      const int64_t t = r % a.Q;
      const int64_t ch = c0 + cc;
      Acc f = 0;
      if (t < n && ch < nc && ch * a.C <= len + t) {
        const Acc mc = static_cast<Acc>(chunk_ml[(ch * a.R + r) * 2]);
        f = mc == neg_inf ? Acc(0) : acc_exp(mc - row_m[i]) * row_inv_l[i];
      }
      fac[i][cc] = f;
    }
    __syncthreads();
    // 3. rescale visible slots, zero the rest
    if (vec) {
      for (int64_t base = e0 + tid * 8; base < e1; base += kCombineThreads * 8) {
        const int cc = static_cast<int>((base - e0) / a.C);
        Vec8<T> x[RB];
#pragma unroll
        for (int i = 0; i < RB; i++) {
          if (i < nrows) {
            const int r = rb + i;
            const int64_t g = r / a.Q, t = r % a.Q;
            const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
            const int64_t lim = t < n ? len + t + 1 : 0;  // visible slots [0, lim)
            if (base < lim) x[i].load(att + row * a.M + base); else x[i].zero();
          }
        }
#pragma unroll
        for (int i = 0; i < RB; i++) {
          if (i < nrows) {
            const int r = rb + i;
            const int64_t g = r / a.Q, t = r % a.Q;
            const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
            const int64_t lim = t < n ? len + t + 1 : 0;
            if (base < lim) {
              x[i].scale_by(fac[i][cc]);
              // zero the invisible part of this vector
              if (base + 8 > lim) x[i].keep_first(static_cast<int>(lim - base));
            }
            x[i].store(att + row * a.M + base);
          }
        }
      }
    } else {
      for (int i = 0; i < nrows; i++) {
        const int r = rb + i;
        const int64_t g = r / a.Q, t = r % a.Q;
        const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
        const int64_t lim = t < n ? len + t + 1 : 0;
        T* arow = att + row * a.M;
        for (int64_t j = e0 + tid; j < e1; j += kCombineThreads) {
          if (j < lim)
            E::store(arow + j, E::load(arow + j) * fac[i][(j - e0) / a.C]);
          else
            arow[j] = E::zero();
        }
      }
    }
    // 4. context of the rows this range owns: the whole workgroup reduces
    //    one row at a time, segment weights exp(m_seg - m) / l staged in LDS
    for (int i = 0; i < nrows; i++) {
      const int r = rb + i;
      if ((r % ncw) != k) continue;
      const int64_t g = r / a.Q, t = r % a.Q;
      const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
      if (t >= n) {
        for (int64_t dv = tid; dv < a.Dv; dv += kCombineThreads) ctx[row * a.Dv + dv] = E::zero();
        continue;
      }
      // PARTS threads per dv (Dv < 256) each sum every PARTS-th segment
      const int parts = a.Dv >= kCombineThreads ? 1 : kCombineThreads / static_cast<int>(a.Dv);
      for (int64_t dv0 = 0; dv0 < a.Dv; dv0 += kCombineThreads) {
        const int64_t dv = dv0 + tid % (parts == 1 ? kCombineThreads : a.Dv);
        const int part = parts == 1 ? 0 : tid / static_cast<int>(a.Dv);
        Acc o = 0;
        for (int64_t s0 = 0; s0 < sr.count; s0 += kCombineThreads) {
          const int64_t ns = sr.count - s0 < kCombineThreads ? sr.count - s0 : kCombineThreads;
          __syncthreads();
          if (tid < ns) {
            const Acc mk = static_cast<Acc>(a.ws_seg_ml[((sr.first + s0 + tid) * a.R + r) * 2]);
            seg_w[tid] = mk == neg_inf ? Acc(0) : acc_exp(mk - row_m[i]) * row_inv_l[i];
          }
          __syncthreads();
          if (part < parts && dv < a.Dv) {
            const float* op = a.ws_seg_o + ((sr.first + s0) * a.R + r) * a.Dv + dv;
#pragma unroll 4
            for (int64_t s = part; s < ns; s += parts) o += seg_w[s] * static_cast<Acc>(op[s * a.R * a.Dv]);
          }
        }
        __syncthreads();
        ctx_red[tid] = part < parts ? o : Acc(0);  // slot tid = part * Dv + dv (parts > 1)
        __syncthreads();
        if (tid < (parts == 1 ? kCombineThreads : a.Dv) && dv0 + tid < a.Dv) {
          Acc sum = 0;
          for (int p = 0; p < parts; p++) sum += ctx_red[p * (parts == 1 ? 0 : a.Dv) + tid];
          E::store(ctx + row * a.Dv + dv0 + tid, sum);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace kvc
