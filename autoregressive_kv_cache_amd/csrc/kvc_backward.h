// kvc_backward.h -- backward of the step for fp32 inputs: the gradients of
// the query, the appended rows and the cache given those of the outputs
// (attention, context, and the returned caches).  The page "Autoregressive
// KV-cache append and causal attention" grades gradients too (its workspace
// note); the forward is the one of Required behavior, so with K', V' the
// updated caches, P the attention rows and O the context of a valid row:
//   dP_j = dA_j + dO . V'_j,   dS_j = P_j (dP_j - sum_k P_k dP_k),
//   dq   = scale sum_j dS_j K'_j,
//   dK'_j += scale dS_j q,     dV'_j += P_j dO,
// and dK' / dV' split into the cache slots that were kept (-> the cache
// gradient, plus the returned cache's gradient passed through) and the
// slots that were overwritten (-> the appended rows' gradient; the old
// cache entry gets none).  Rows outside the contract are no-ops: only the
// pass-through remains.
//
// Precision: fp32 inputs reach scores near 1e3, where P is nearly one-hot
// and dP_j - sum_k P_k dP_k cancels; so P is recomputed from the scores
// with the row's max and sum in fp64 (as the forward keeps its statistics),
// dP and that sum are formed in fp64, and the query gradient is summed in
// fp64.  The forward's fp32 attention and context are not needed.
//
// Kernels: bwd_stats (one workgroup per (b, KV head, 64-slot chunk): each
// packed row's max, sum and sum of P dP over the chunk's slots, K' and V'
// staged once for all rows of the head), bwd_rows (one wave per packed
// row: the chunk statistics merged as the forward merges its segments),
// bwd_chunk (same grid as bwd_stats: dS for the chunk's slots and all
// packed rows, the slot gradients, and per-chunk dq partials), bwd_dq (one
// wave per packed row: the partials summed).
#pragma once

#include "kvc_common.h"

namespace kvc {

constexpr int kBwdThreads = 256;
constexpr int kBwdSlots = 64;   // slots per chunk workgroup
constexpr int kBwdRowTile = 16; // packed rows staged in LDS at a time

struct BwdArgs {
  int64_t B, Hq, Hk, Q, M, D, Dv;
  int32_t G, R;
  int64_t nchunk;  // ceil(M / kBwdSlots)
  float scale;
  const float* query;      // [B][Hq][Q][D]
  const float* new_key;    // [B][Hk][Q][D]
  const float* new_value;  // [B][Hk][Q][Dv]
  const float* kc;         // [B][Hk][M][D]: slots < length (the updated cache or the old one)
  const float* vc;
  const int64_t* lengths;  // the step's input lengths
  const uint8_t* mask;
  const float* d_att;      // gradients of the outputs (null = zero)
  const float* d_ctx;
  const float* d_kc_out;   // [B][Hk][M][D]
  const float* d_vc_out;
  float* g_query;          // gradients of the inputs
  float* g_new_key;
  float* g_new_value;
  float* g_kc;
  float* g_vc;
  double* ws_row;          // [B][Hq][Q][4]: m, l, sum_k P_k dP_k / l
  double* ws_part;         // [B*Hk][nchunk][R][4]: m_c, l_c, sum over the chunk of e^(s-m_c) dP
  double* ws_dq;           // [B*Hk][nchunk][R][D]
};

// Row information of batch row b for one thread (prefix count n, status).
__device__ inline void bwd_row_info(const BwdArgs& a, int64_t b, int64_t* len, int64_t* n) {
  const int64_t L = a.lengths[b];
  int64_t k = 0;
  while (k < a.Q && a.mask[b * a.Q + k]) k++;
  bool ok = L >= 0 && L <= a.M && L + k <= a.M;
  for (int64_t t = k; t < a.Q; t++) ok = ok && !a.mask[b * a.Q + t];
  *len = L;
  *n = ok ? k : 0;
}

// fp64 dot product of two fp32 vectors of length N (a multiple of 4), as
// four independent partial sums so that consecutive FMAs do not wait on
// each other.
template <int N>
__device__ __forceinline__ double dot_f64(const float* x, const float* y) {
  static_assert(N % 4 == 0, "length");
  double s0 = 0, s1 = 0, s2 = 0, s3 = 0;
#pragma unroll 4
  for (int d = 0; d < N; d += 4) {
    s0 += static_cast<double>(x[d]) * y[d];
    s1 += static_cast<double>(x[d + 1]) * y[d + 1];
    s2 += static_cast<double>(x[d + 2]) * y[d + 2];
    s3 += static_cast<double>(x[d + 3]) * y[d + 3];
  }
  return (s0 + s1) + (s2 + s3);
}

// Slot j of the updated caches: kept rows from the cache, appended rows
// (j >= len) from new_key / new_value.
__device__ inline const float* bwd_key_row(const BwdArgs& a, int64_t grp, int64_t len, int64_t j) {
  return j < len ? a.kc + (grp * a.M + j) * a.D : a.new_key + (grp * a.Q + (j - len)) * a.D;
}
__device__ inline const float* bwd_value_row(const BwdArgs& a, int64_t grp, int64_t len,
                                             int64_t j) {
  return j < len ? a.vc + (grp * a.M + j) * a.Dv : a.new_value + (grp * a.Q + (j - len)) * a.Dv;
}

// One workgroup per (b, KV head, chunk of kBwdSlots slots): for every valid
// packed row, over the chunk's slots it sees, m_c = max s_j, l_c =
// sum e^(s_j - m_c) and sum e^(s_j - m_c) dP_j, in fp64 (one wave per row,
// one lane per slot).
template <int D, int DV>
__global__ __launch_bounds__(kBwdThreads) void bwd_stats_kernel(BwdArgs a) {
  constexpr int C = kBwdSlots, RT = kBwdRowTile, W = kBwdThreads / kWave;
  static_assert(C == kWave, "one lane per slot");
  __shared__ float k_s[C][D + 1];
  __shared__ float v_s[C][DV + 1];
  __shared__ float q_s[RT][D + 1];
  __shared__ float o_s[RT][DV + 1];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int64_t c = blockIdx.x % a.nchunk;
  const int64_t grp = blockIdx.x / a.nchunk;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  const int64_t s0 = c * C;
  const int64_t nvis = n > 0 ? len + n : 0;
  if (s0 >= nvis) return;  // no row sees this chunk
  for (int idx = tid; idx < C * D; idx += kBwdThreads) {
    const int sl = idx / D, d = idx % D;
    const int64_t j = s0 + sl;
    k_s[sl][d] = j < nvis ? bwd_key_row(a, grp, len, j)[d] : 0.f;
  }
  for (int idx = tid; idx < C * DV; idx += kBwdThreads) {
    const int sl = idx / DV, d = idx % DV;
    const int64_t j = s0 + sl;
    v_s[sl][d] = j < nvis ? bwd_value_row(a, grp, len, j)[d] : 0.f;
  }
  const int64_t j = s0 + lane;
  for (int r0 = 0; r0 < a.R; r0 += RT) {
    __syncthreads();
    for (int idx = tid; idx < RT * D; idx += kBwdThreads) {
      const int rr = idx / D, d = idx % D, r = r0 + rr;
      const int64_t g = r / a.Q, t = r % a.Q;
      q_s[rr][d] = (r < a.R && t < n)
                       ? a.query[((b * a.Hq + kvh * a.G + g) * a.Q + t) * D + d] : 0.f;
    }
    for (int idx = tid; idx < RT * DV; idx += kBwdThreads) {
      const int rr = idx / DV, d = idx % DV, r = r0 + rr;
      const int64_t g = r / a.Q, t = r % a.Q;
      o_s[rr][d] = (a.d_ctx && r < a.R && t < n)
                       ? a.d_ctx[((b * a.Hq + kvh * a.G + g) * a.Q + t) * DV + d] : 0.f;
    }
    __syncthreads();
    for (int rr = wave; rr < RT; rr += W) {
      const int r = r0 + rr;
      if (r >= a.R) break;
      const int64_t g = r / a.Q, t = r % a.Q;
      if (t >= n) continue;
      const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
      const bool vis = j <= len + t;
      double sc = 0, dp = 0;
      if (vis) {
        sc = static_cast<double>(a.scale) * dot_f64<D>(q_s[rr], k_s[lane]);
        dp = (a.d_att ? static_cast<double>(a.d_att[row * a.M + j]) : 0.0) +
             dot_f64<DV>(o_s[rr], v_s[lane]);
      }
      double m = vis ? sc : -INFINITY;
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const double y = __shfl_xor(m, o);
        m = y > m ? y : m;
      }
      const double e = vis ? exp(sc - m) : 0.0;
      double l = e, pd = e * dp;
      for (int o = kWave / 2; o > 0; o >>= 1) {
        l += __shfl_xor(l, o);
        pd += __shfl_xor(pd, o);
      }
      if (lane == 0) {
        double* out = a.ws_part + ((grp * a.nchunk + c) * a.R + r) * 4;
        out[0] = m;
        out[1] = l;
        out[2] = pd;
        out[3] = 0.0;
      }
    }
  }
}

// One wave per packed row: its chunk statistics merged (m = max m_c,
// l = sum l_c e^(m_c - m), the same for the P dP sums), then divided by l.
__global__ __launch_bounds__(kBwdThreads) void bwd_rows_kernel(BwdArgs a) {
  const int64_t row = blockIdx.x * (kBwdThreads / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= a.B * a.Hq * a.Q) return;
  const int64_t t = row % a.Q, hq = (row / a.Q) % a.Hq, b = row / (a.Hq * a.Q);
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  const int64_t kvh = hq / a.G, g = hq % a.G, r = g * a.Q + t, grp = b * a.Hk + kvh;
  const int64_t nc = t < n ? (len + t) / kBwdSlots + 1 : 0;
  double m = -INFINITY, l = 0, pd = 0;
  for (int64_t c = lane; c < nc; c += kWave) {
    const double* p = a.ws_part + ((grp * a.nchunk + c) * a.R + r) * 4;
    const double mn = p[0] > m ? p[0] : m;
    const double fo = m == -INFINITY ? 0.0 : exp(m - mn), fn = exp(p[0] - mn);
    l = l * fo + p[1] * fn;
    pd = pd * fo + p[2] * fn;
    m = mn;
  }
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const double mo = __shfl_xor(m, o), lo = __shfl_xor(l, o), po = __shfl_xor(pd, o);
    const double mn = mo > m ? mo : m;
    if (mn != -INFINITY) {
      const double fa = m == -INFINITY ? 0.0 : exp(m - mn);
      const double fb = mo == -INFINITY ? 0.0 : exp(mo - mn);
      l = l * fa + lo * fb;
      pd = pd * fa + po * fb;
    }
    m = mn;
  }
  if (lane == 0) {
    double* out = a.ws_row + row * 4;
    out[0] = nc > 0 ? m : 0.0;
    out[1] = nc > 0 ? l : 0.0;
    out[2] = nc > 0 ? pd / l : 0.0;
    out[3] = 0.0;
  }
}

// One workgroup per (b, KV head, chunk of kBwdSlots slots).
template <int D, int DV>
__global__ __launch_bounds__(kBwdThreads) void bwd_chunk_kernel(BwdArgs a) {
  constexpr int C = kBwdSlots, RT = kBwdRowTile;
  __shared__ float k_s[C][D + 1];
  __shared__ float v_s[C][DV + 1];
  __shared__ float q_s[RT][D + 1];
  __shared__ float o_s[RT][DV + 1];   // dO rows
  __shared__ double ds_s[RT][C + 1];  // scale * dS
  __shared__ float p_s[RT][C + 1];    // P (0 where not visible)
  const int tid = threadIdx.x;
  const int64_t c = blockIdx.x % a.nchunk;
  const int64_t grp = blockIdx.x / a.nchunk;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  const int64_t s0 = c * C;
  // slots with any attention gradient (none on a row that appends nothing
  // or is rejected; then only the pass-through below remains)
  const int64_t nvis = n > 0 ? len + n : 0;

  // K', V' rows of the chunk (zeros past the visible slots)
  for (int idx = tid; idx < C * D; idx += kBwdThreads) {
    const int s = idx / D, d = idx % D;
    const int64_t j = s0 + s;
    float x = 0.f;
    if (j < nvis)
      x = j < len ? a.kc[((grp * a.M) + j) * D + d] : a.new_key[(grp * a.Q + (j - len)) * D + d];
    k_s[s][d] = x;
  }
  for (int idx = tid; idx < C * DV; idx += kBwdThreads) {
    const int s = idx / DV, d = idx % DV;
    const int64_t j = s0 + s;
    float x = 0.f;
    if (j < nvis)
      x = j < len ? a.vc[((grp * a.M) + j) * DV + d]
                  : a.new_value[(grp * a.Q + (j - len)) * DV + d];
    v_s[s][d] = x;
  }

  // slot gradients: thread owns (slot, dim) pairs of dK' and dV'
  constexpr int KPT = (C * D + kBwdThreads - 1) / kBwdThreads;
  constexpr int VPT = (C * DV + kBwdThreads - 1) / kBwdThreads;
  float gk[KPT], gv[VPT];
#pragma unroll
  for (int i = 0; i < KPT; i++) gk[i] = 0.f;
#pragma unroll
  for (int i = 0; i < VPT; i++) gv[i] = 0.f;

  const bool any = s0 < nvis;  // nvis <= M
  for (int r0 = 0; any && r0 < a.R; r0 += RT) {
    __syncthreads();  // the previous tile's LDS is no longer read
    for (int idx = tid; idx < RT * D; idx += kBwdThreads) {
      const int rr = idx / D, d = idx % D, r = r0 + rr;
      const int64_t g = r / a.Q, t = r % a.Q;
      q_s[rr][d] = (r < a.R && t < n)
                       ? a.query[((b * a.Hq + kvh * a.G + g) * a.Q + t) * D + d] : 0.f;
    }
    for (int idx = tid; idx < RT * DV; idx += kBwdThreads) {
      const int rr = idx / DV, d = idx % DV, r = r0 + rr;
      const int64_t g = r / a.Q, t = r % a.Q;
      o_s[rr][d] = (a.d_ctx && r < a.R && t < n)
                       ? a.d_ctx[((b * a.Hq + kvh * a.G + g) * a.Q + t) * DV + d] : 0.f;
    }
    __syncthreads();
    // dS for (row, slot), in fp64: P from the score and the row's m, l;
    // dP = dA + dO . V'_j
    for (int idx = tid; idx < RT * C; idx += kBwdThreads) {
      const int rr = idx / C, s = idx % C, r = r0 + rr;
      const int64_t g = r / a.Q, t = r % a.Q, j = s0 + s;
      double ds = 0, p = 0;
      if (r < a.R && t < n && j <= len + t) {
        const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
        const double* st = a.ws_row + row * 4;
        const double sc = dot_f64<D>(q_s[rr], k_s[s]);
        p = exp(static_cast<double>(a.scale) * sc - st[0]) / st[1];
        const double dp = (a.d_att ? static_cast<double>(a.d_att[row * a.M + j]) : 0.0) +
                          dot_f64<DV>(o_s[rr], v_s[s]);
        ds = static_cast<double>(a.scale) * p * (dp - st[2]);
      }
      ds_s[rr][s] = ds;
      p_s[rr][s] = static_cast<float>(p);
    }
    __syncthreads();
    // dK'_j += sum_r ds q_r, dV'_j += sum_r p dO_r
#pragma unroll
    for (int i = 0; i < KPT; i++) {
      const int idx = tid + i * kBwdThreads;
      if (idx < C * D) {
        const int s = idx / D, d = idx % D;
        float acc = gk[i];
        for (int rr = 0; rr < RT; rr++) acc += static_cast<float>(ds_s[rr][s]) * q_s[rr][d];
        gk[i] = acc;
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; i++) {
      const int idx = tid + i * kBwdThreads;
      if (idx < C * DV) {
        const int s = idx / DV, d = idx % DV;
        float acc = gv[i];
        for (int rr = 0; rr < RT; rr++) acc += p_s[rr][s] * o_s[rr][d];
        gv[i] = acc;
      }
    }
    // dq partial of this chunk: sum_j ds_j K'_j
    for (int idx = tid; idx < RT * D; idx += kBwdThreads) {
      const int rr = idx / D, d = idx % D, r = r0 + rr;
      if (r >= a.R) continue;
      double acc0 = 0, acc1 = 0;
      for (int s = 0; s < C; s += 2) {
        acc0 += ds_s[rr][s] * k_s[s][d];
        acc1 += ds_s[rr][s + 1] * k_s[s + 1][d];
      }
      a.ws_dq[((grp * a.nchunk + c) * a.R + r) * D + d] = acc0 + acc1;
    }
  }

  // slot gradients out: kept slots -> the cache gradient, overwritten ones
  // -> the appended rows' gradient (the cache entry gets 0), the rest ->
  // the pass-through alone
#pragma unroll
  for (int i = 0; i < KPT; i++) {
    const int idx = tid + i * kBwdThreads;
    if (idx < C * D) {
      const int s = idx / D, d = idx % D;
      const int64_t j = s0 + s;
      if (j < a.M) {
        const int64_t at = (grp * a.M + j) * D + d;
        const float total = gk[i] + (a.d_kc_out ? a.d_kc_out[at] : 0.f);
        if (j >= len && j < len + n) {
          a.g_new_key[(grp * a.Q + (j - len)) * D + d] = total;
          a.g_kc[at] = 0.f;
        } else {
          a.g_kc[at] = total;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < VPT; i++) {
    const int idx = tid + i * kBwdThreads;
    if (idx < C * DV) {
      const int s = idx / DV, d = idx % DV;
      const int64_t j = s0 + s;
      if (j < a.M) {
        const int64_t at = (grp * a.M + j) * DV + d;
        const float total = gv[i] + (a.d_vc_out ? a.d_vc_out[at] : 0.f);
        if (j >= len && j < len + n) {
          a.g_new_value[(grp * a.Q + (j - len)) * DV + d] = total;
          a.g_vc[at] = 0.f;
        } else {
          a.g_vc[at] = total;
        }
      }
    }
  }
  // appended rows that do not exist (t >= n, rejected rows): zero gradient
  if (c == 0) {
    for (int64_t idx = tid; idx < (a.Q - n) * D; idx += kBwdThreads)
      a.g_new_key[(grp * a.Q + n + idx / D) * D + idx % D] = 0.f;
    for (int64_t idx = tid; idx < (a.Q - n) * DV; idx += kBwdThreads)
      a.g_new_value[(grp * a.Q + n + idx / DV) * DV + idx % DV] = 0.f;
  }
}

// dq_r = sum over the chunks its row can see of the partials (0 for rows
// that are not valid).
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(BwdArgs a) {
  const int64_t row = blockIdx.x * (kBwdThreads / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= a.B * a.Hq * a.Q) return;
  const int64_t t = row % a.Q, hq = (row / a.Q) % a.Hq, b = row / (a.Hq * a.Q);
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  const int64_t kvh = hq / a.G, g = hq % a.G, r = g * a.Q + t, grp = b * a.Hk + kvh;
  const int64_t nc = t < n ? (len + t) / kBwdSlots + 1 : 0;  // chunks holding slots <= len + t
  for (int64_t d = lane; d < a.D; d += kWave) {
    double acc = 0;
    for (int64_t c = 0; c < nc; c++) acc += a.ws_dq[((grp * a.nchunk + c) * a.R + r) * a.D + d];
    a.g_query[row * a.D + d] = static_cast<float>(acc);
  }
}

}  // namespace kvc
