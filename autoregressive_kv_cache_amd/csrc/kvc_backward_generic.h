// kvc_backward_generic.h -- backward of the step for any head sizes (D, Dv)
// and any element-aligned buffers: the shapes the tiled kernels of
// kvc_backward.h and kvc_backward_vec.h do not take (head sizes without a
// compiled tile, or buffers that are not 16-byte aligned).  The math is the
// one of kvc_backward.h ("Autoregressive KV-cache append and causal
// attention", Required behavior, differentiated):
//   dP_j = dA_j + dO . V'_j,   dS_j = P_j (dP_j - sum_k P_k dP_k),
//   dq = scale sum_j dS_j K'_j, dK'_j += scale dS_j q, dV'_j += P_j dO,
// here with every dot product, softmax term and sum in fp64 and each
// gradient rounded once to the element type.
//
// Kernels (one workgroup per (b, KV head, 64-slot chunk); the partials
// have the layout of kvc_backward.h's, so bwd_rows_kernel merges them):
//   bwd_gstats: per packed row, the chunk's max score, sum of exp(s - m_c)
//     and sum of exp(s - m_c) dP;
//   bwd_gchunk: the chunk in pieces of CS slots (CS a power of two chosen so
//     that a piece's slot accumulators fit the LDS); per piece and packed
//     row tile, P and dS, the tile's dq partials, and dK', dV' summed over
//     every row in LDS, then stored with the returned caches' gradients
//     added (kept slots to the cache gradient, appended ones to the new
//     rows'); slots no row sees get the pass-through as it is;
//   bwd_gdq: per packed row, its dq partials summed.
// Element loads are scalar, so no alignment beyond the element's is needed.
#pragma once

#include "kvc_backward.h"

namespace kvc {

constexpr int kBwdGenRows = 16;                 // packed rows per tile
constexpr int kBwdGenAccDoubles = 6144;         // slot accumulators: C (D + Dv) <= this

// Slots per piece for head sizes D, Dv: the largest power of two <= 64
// with C (D + Dv) accumulators in kBwdGenAccDoubles (48 KiB); 0 when
// D + Dv is too large even for one slot.
__host__ __device__ inline int bwd_gen_slots(int64_t D, int64_t Dv) {
  const int64_t w = D + Dv;
  if (w > kBwdGenAccDoubles) return 0;
  int c = 64;
  while (c > 1 && static_cast<int64_t>(c) * w > kBwdGenAccDoubles) c /= 2;
  return c;
}

template <typename T>
__device__ __forceinline__ double bwd_gld(const void* p, int64_t i) {
  return static_cast<double>(bwd_ld<T>(p, i));
}

__device__ __forceinline__ double bwd_wave_max_d(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const double w = __shfl_xor(v, o);
    v = v > w ? v : w;
  }
  return v;
}
__device__ __forceinline__ double bwd_wave_sum_d(double v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// (b, query head, token) row of packed row r of KV head kvh
__device__ __forceinline__ int64_t bwd_gen_qrow(const BwdArgs& a, int64_t b, int64_t kvh, int r) {
  return (b * a.Hq + kvh * a.G + r / a.Q) * a.Q + r % a.Q;
}

// Score and dP of packed row r against slot j (visible: fp64 dots; else
// s = -inf, dP = 0).
template <typename T>
__device__ inline void bwd_gen_pair(const BwdArgs& a, int64_t b, int64_t kvh, int64_t grp,
                                    int64_t len, int64_t n, int r, int64_t j, double* s,
                                    double* dp) {
  const int64_t t = r % a.Q;
  *s = -INFINITY;
  *dp = 0.0;
  if (!(t < n && j <= len + t)) return;
  const int64_t qr = bwd_gen_qrow(a, b, kvh, r);
  int64_t ko = 0, vo = 0;
  const void* kp = bwd_key_src(a, grp, len, j, &ko);
  const void* vp = bwd_value_src(a, grp, len, j, &vo);
  double dot = 0.0;
  for (int64_t d = 0; d < a.D; d++) dot += bwd_gld<T>(a.query, qr * a.D + d) * bwd_gld<T>(kp, ko + d);
  double g = a.d_att ? bwd_gld<T>(a.d_att, qr * a.M + j) : 0.0;
  if (a.d_ctx)
    for (int64_t d = 0; d < a.Dv; d++)
      g += bwd_gld<T>(a.d_ctx, qr * a.Dv + d) * bwd_gld<T>(vp, vo + d);
  *s = a.scale_d * dot;
  *dp = g;
}

template <typename T>
__global__ __launch_bounds__(kBwdThreads) void bwd_gstats_kernel(BwdArgs a) {
  constexpr int RT = kBwdGenRows, W = kBwdThreads / kWave;
  __shared__ double s_sh[RT][64], p_sh[RT][64];
  const int C = a.part_slots, tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t c = blockIdx.x % a.nchunk, grp = blockIdx.x / a.nchunk;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk, s0 = c * C;
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  if (n == 0 || s0 >= len + n) return;  // no row sees a slot of this chunk
  for (int r0 = 0; r0 < a.R; r0 += RT) {
    const int rc = a.R - r0 < RT ? a.R - r0 : RT;
    for (int idx = tid; idx < rc * C; idx += kBwdThreads) {
      double s, dp;
      bwd_gen_pair<T>(a, b, kvh, grp, len, n, r0 + idx / C, s0 + idx % C, &s, &dp);
      s_sh[idx / C][idx % C] = s;
      p_sh[idx / C][idx % C] = dp;
    }
    __syncthreads();
    for (int rr = wave; rr < rc; rr += W) {
      const double s = lane < C ? s_sh[rr][lane] : -INFINITY;
      const double m = bwd_wave_max_d(s);
      const double e = (s == -INFINITY) ? 0.0 : exp(s - m);
      const double l = bwd_wave_sum_d(e);
      const double pd = bwd_wave_sum_d(lane < C ? e * p_sh[rr][lane] : 0.0);
      if (lane == 0) {
        double* out = a.ws_part + ((grp * a.nchunk + c) * a.R + r0 + rr) * 4;
        out[0] = m;
        out[1] = l;
        out[2] = pd;
        out[3] = 0.0;
      }
    }
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(kBwdThreads) void bwd_gchunk_kernel(BwdArgs a) {
  constexpr int RT = kBwdGenRows;
  extern __shared__ double acc[];  // [CS][D] key gradients, then [CS][Dv] value gradients
  __shared__ double P_sh[RT][64], dS_sh[RT][64];
  const int CS = a.gen_slots, tid = threadIdx.x;
  const int64_t D = a.D, Dv = a.Dv, WD = D + Dv;
  const int64_t c = blockIdx.x % a.nchunk, grp = blockIdx.x / a.nchunk;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk, s0 = c * a.part_slots;
  const int64_t s_end = s0 + a.part_slots < a.M ? s0 + a.part_slots : a.M;
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);

  if (c == 0)  // new rows that were not appended get no gradient
    for (int64_t i = tid; i < (a.Q - n) * WD; i += kBwdThreads) {
      const int64_t t = n + i / WD, e = i % WD;
      if (e < D)
        bwd_st<T>(a.g_new_key, (grp * a.Q + t) * D + e, 0.f);
      else
        bwd_st<T>(a.g_new_value, (grp * a.Q + t) * Dv + (e - D), 0.f);
    }

  // the chunk's slots in pieces of CS (the accumulators of one piece fit the
  // LDS); a thread keeps the same accumulator entries, and the same dq
  // partial entries, from piece to piece, so only P / dS need barriers
  for (int64_t sub = s0; sub < s_end; sub += CS) {
    const bool touched = n > 0 && sub < len + n;  // some row sees a slot of the piece
    if (touched) {
      for (int64_t i = tid; i < CS * WD; i += kBwdThreads) acc[i] = 0.0;
      const int64_t jn = len + n - sub < CS ? len + n - sub : CS;  // slots below len + n
      for (int r0 = 0; r0 < a.R; r0 += RT) {
        const int rc = a.R - r0 < RT ? a.R - r0 : RT;
        for (int idx = tid; idx < rc * CS; idx += kBwdThreads) {
          const int r = r0 + idx / CS;
          double s, dp;
          bwd_gen_pair<T>(a, b, kvh, grp, len, n, r, sub + idx % CS, &s, &dp);
          double P = 0.0, dS = 0.0;
          if (s != -INFINITY) {
            const double* st = a.ws_row + bwd_gen_qrow(a, b, kvh, r) * 4;
            P = exp(s - st[0]) / st[1];
            dS = P * (dp - st[2]);
          }
          P_sh[idx / CS][idx % CS] = P;
          dS_sh[idx / CS][idx % CS] = dS;
        }
        __syncthreads();
        // dq partials of the tile's rows: scale sum_j dS_j K'_j over the
        // chunk, the first piece storing and the later ones adding
        for (int64_t idx = tid; idx < rc * D; idx += kBwdThreads) {
          const int rr = static_cast<int>(idx / D);
          const int64_t d = idx % D;
          double sum = 0.0;
          for (int jj = 0; jj < jn; jj++) {
            int64_t ko = 0;
            const void* kp = bwd_key_src(a, grp, len, sub + jj, &ko);
            sum += dS_sh[rr][jj] * bwd_gld<T>(kp, ko + d);
          }
          double* at = a.ws_dq + ((grp * a.nchunk + c) * a.R + r0 + rr) * D + d;
          *at = (sub == s0 ? 0.0 : *at) + a.scale_d * sum;
        }
        // slot gradients: dK'_j += scale sum_r dS_jr q_r, dV'_j += sum_r P_jr dO_r
        for (int64_t idx = tid; idx < CS * WD; idx += kBwdThreads) {
          const int jj = static_cast<int>(idx / WD);
          const int64_t e = idx % WD;
          double sum = 0.0;
          if (e < D) {
            for (int rr = 0; rr < rc; rr++)
              if (dS_sh[rr][jj] != 0.0)
                sum += dS_sh[rr][jj] *
                       bwd_gld<T>(a.query, bwd_gen_qrow(a, b, kvh, r0 + rr) * D + e);
            acc[idx] += a.scale_d * sum;
          } else if (a.d_ctx) {
            for (int rr = 0; rr < rc; rr++)
              if (P_sh[rr][jj] != 0.0)
                sum += P_sh[rr][jj] *
                       bwd_gld<T>(a.d_ctx, bwd_gen_qrow(a, b, kvh, r0 + rr) * Dv + (e - D));
            acc[idx] += sum;
          }
        }
        __syncthreads();
      }
    }
    // store: slot j of the piece, element e of its key (e < D) or value row
    for (int64_t idx = tid; idx < CS * WD; idx += kBwdThreads) {
      const int64_t j = sub + idx / WD, e = idx % WD;
      if (j >= s_end) continue;
      const bool key = e < D;
      const int64_t w = key ? D : Dv, col = key ? e : e - D;
      const void* pass = key ? a.d_kc_out : a.d_vc_out;
      void* gcache = key ? a.g_kc : a.g_vc;
      const int64_t at = (grp * a.M + j) * w + col;
      if (!touched || j >= len + n) {  // no row sees the slot: the pass-through as it is
        if constexpr (sizeof(T) == 2)
          static_cast<uint16_t*>(gcache)[at] = pass ? static_cast<const uint16_t*>(pass)[at] : 0;
        else
          static_cast<float*>(gcache)[at] = pass ? static_cast<const float*>(pass)[at] : 0.f;
        continue;
      }
      const double g = (pass ? bwd_gld<T>(pass, at) : 0.0) + acc[idx];
      if (j >= len) {  // appended: its gradient goes to the new row, the old entry gets none
        bwd_st<T>(key ? a.g_new_key : a.g_new_value, (grp * a.Q + (j - len)) * w + col,
                  static_cast<float>(g));
        bwd_st<T>(gcache, at, 0.f);
      } else {
        bwd_st<T>(gcache, at, static_cast<float>(g));
      }
    }
  }
}

// dq_r = the sum of its row's partials over the chunks it can see (0 for a
// row that is not valid).  One workgroup per row, a thread per column.
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void bwd_gdq_kernel(BwdArgs a) {
  const int64_t row = blockIdx.x;
  const int64_t t = row % a.Q, hq = (row / a.Q) % a.Hq, b = row / (a.Hq * a.Q);
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  const int64_t kvh = hq / a.G, g = hq % a.G, r = g * a.Q + t, grp = b * a.Hk + kvh;
  const int64_t nc = t < n ? (len + t) / a.part_slots + 1 : 0;
  for (int64_t d = threadIdx.x; d < a.D; d += kBwdThreads) {
    double sum = 0.0;
    for (int64_t c = 0; c < nc; c++) sum += a.ws_dq[((grp * a.nchunk + c) * a.R + r) * a.D + d];
    bwd_st<T>(a.g_query, row * a.D + d, static_cast<float>(sum));
  }
}

}  // namespace kvc
