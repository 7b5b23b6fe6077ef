// kvc_small.h -- decode-path attend kernel for small heads: rows of at most
// 64 bytes (fp32 D, Dv <= 16; bf16 <= 32), where the decode kernel's layout
// (several lanes per K row, one finished dot product per lane) has fewer
// lanes per row than packed rows.  Here one lane holds one slot's whole K
// and V rows, so every dot product finishes in its lane; the per-row chunk
// statistics and the segment's context are summed across the wave.
//
// Work split, workspace and outputs are those of attend_decode_kernel
// (kvc_decode.h), so the same combine kernel follows: the visible slots of
// every (batch row, KV head) in chunks of 64 slots -- the cached slots, then
// one chunk with the appended rows read from new_key / new_value -- and the
// flattened chunk list cut into contiguous ranges, one per wave; per chunk
// exp(s - m_c) into the attention rows and (m_c, l_c) into the workspace; per
// segment (the chunks of one KV head in a wave's range) its statistics and
// unnormalised context.  Scores are scale * dot(q, k) over j <= length + t
// ("Autoregressive KV-cache append and causal attention", Required behavior;
// the lower-right alignment of KempnerForge PR 542, Summary), in fp64 for
// fp32 tensors and fp32 for bf16 (DecodeMath).
#pragma once

#include "kvc_decode.h"
#include "kvc_stream.h"

namespace kvc {

constexpr int kSmallChunk = kWave;  // one slot per lane

// Max or sum over all 64 lanes, every lane getting the result: row
// rotations (DPP) inside each 16-lane row, then the permlane16 / permlane32
// swaps across rows (wave_reduce of kvc_stream.h for fp32; the same steps
// on both halves of an fp64 value here).
// The permlane swaps with both operands v: one result holds this lane's
// value, the other its partner's (lane bit 4 or 5 flipped); both halves of
// an fp64 value travel the same way, so (a, b) are whole values.
template <bool ACROSS32>
__device__ __forceinline__ void swap_pair(double v, double* a, double* b) {
  const int2 w = __builtin_bit_cast(int2, v);
  const uint32_t x = static_cast<uint32_t>(w.x), y = static_cast<uint32_t>(w.y);
  const auto lo = ACROSS32 ? __builtin_amdgcn_permlane32_swap(x, x, false, false)
                           : __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const auto hi = ACROSS32 ? __builtin_amdgcn_permlane32_swap(y, y, false, false)
                           : __builtin_amdgcn_permlane16_swap(y, y, false, false);
  *a = __builtin_bit_cast(double, make_int2(static_cast<int>(lo[0]), static_cast<int>(hi[0])));
  *b = __builtin_bit_cast(double, make_int2(static_cast<int>(lo[1]), static_cast<int>(hi[1])));
}
template <bool MAX>
__device__ __forceinline__ double small_reduce(double v) {
  auto op = [](double x, double y) { return MAX ? (x > y ? x : y) : x + y; };
  v = op(v, dpp<dpp_row_ror(8)>(v));
  v = op(v, dpp<dpp_row_ror(4)>(v));
  v = op(v, dpp<dpp_row_ror(2)>(v));
  v = op(v, dpp<dpp_row_ror(1)>(v));
  double a, b;
  swap_pair<false>(v, &a, &b);
  v = op(a, b);
  swap_pair<true>(v, &a, &b);
  return op(a, b);
}
template <bool MAX>
__device__ __forceinline__ float small_reduce(float v) {
  return wave_reduce<MAX>(v);
}

// Sum of N per-lane values over the wave, scattered: each exchange step
// halves the values a lane holds (lanes with the step's lane bit set keep
// the upper half and add their partner's copy of it), over lane bits 5
// (permlane32 swap), 4 (permlane16 swap) and 3..0 (lane shuffles).  After
// the six steps lane l holds values [l * N / 64, +N / 64) when N >= 64, or
// value l / (64 / N) (summed over the lanes that share it) when N < 64.
template <int N, int BIT>
__device__ __forceinline__ void sum_scatter_step(float (&v)[N], int lane) {
  constexpr int n = (N >> (5 - BIT)) > 0 ? (N >> (5 - BIT)) : 1;  // values held before the step
  if constexpr (n > 1) {
    constexpr int h = n / 2;
    const bool up = (lane >> BIT) & 1;
#pragma unroll
    for (int i = 0; i < h; i++) {
      if constexpr (BIT == 5) {
        v[i] = sum_swap32(v[i], v[h + i]);
      } else if constexpr (BIT == 4) {
        v[i] = sum_swap16(v[i], v[h + i]);
      } else {
        const float give = up ? v[i] : v[h + i];
        v[i] = (up ? v[h + i] : v[i]) + __shfl_xor(give, 1 << BIT);
      }
    }
  } else {
    v[0] += __shfl_xor(v[0], 1 << BIT);
  }
  if constexpr (BIT > 0) sum_scatter_step<N, BIT - 1>(v, lane);
}
template <int N>
__device__ __forceinline__ void sum_scatter(float (&v)[N], int lane) {
  static_assert(N >= 1 && (N & (N - 1)) == 0 && N <= 256, "power of two");
  sum_scatter_step<N, 5>(v, lane);
}

template <typename T, int D, int DV, int ROWS>
__global__ __launch_bounds__(kDecodeThreads) void attend_small_kernel(
    StepArgs a, const int64_t* __restrict__ rowinfo, const int32_t* __restrict__ wstart) {
  using Mth = DecodeMath<T>;
  using Acc = typename Mth::Acc;
  using E = Elem<T>;
  constexpr int C = kSmallChunk;
  constexpr int KROW = D * static_cast<int>(sizeof(T)), VROW = DV * static_cast<int>(sizeof(T));
  constexpr int NK = KROW / 16, NV = VROW / 16;  // 16-byte pieces per row
  static_assert(KROW % 16 == 0 && VROW % 16 == 0 && NK >= 1 && NK <= 4 && NV >= 1 && NV <= 4,
                "rows of 16 to 64 bytes");
  __shared__ int32_t rt_len[kDecodeFusedRows], rt_n[kDecodeFusedRows];
  __shared__ int64_t rt_first[kDecodeFusedRows];
  __shared__ int64_t rt_total;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const bool fused = a.B <= kDecodeFusedRows;
  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  const Acc scale = static_cast<Acc>(a.scale);
  const int Q = static_cast<int>(a.Q), R = static_cast<int>(a.R), Hk = static_cast<int>(a.Hk);
  const int64_t M = a.M;

  // Row information: built in LDS (every workgroup; workgroup 0 publishes
  // it for the combine) for batches of up to kDecodeFusedRows rows, else
  // written by the prep kernel with every worker's start.
  auto row_len = [&](int b) { return fused ? rt_len[b] : static_cast<int>(rowinfo[b * 4 + 0]); };
  auto row_n = [&](int b) { return fused ? rt_n[b] : static_cast<int>(rowinfo[b * 4 + 1]); };
  int64_t Nc, Pw;
  if (fused) {
    for (int b = tid; b < a.B; b += kDecodeThreads) {
      const RowInfo ri = thread_row_info(a.lengths, a.mask, a.Q, a.M, b);
      rt_len[b] = static_cast<int32_t>(ri.len);
      rt_n[b] = static_cast<int32_t>(ri.n);
      if (blockIdx.x == 0) {
        a.ws_rowinfo[b * 4 + 0] = ri.len;
        a.ws_rowinfo[b * 4 + 1] = ri.n;
        a.ws_rowinfo[b * 4 + 2] = ri.status;
      }
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefix of Hk * chunks over the rows
      int64_t carry = 0;
      for (int base = 0; base < a.B; base += kWave) {
        const int b = base + lane;
        const int64_t ch = b < a.B ? Hk * stream_chunks(rt_len[b], rt_n[b], C) : 0;
        int64_t incl = ch;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int64_t up = __shfl_up(incl, o);
          if (lane >= o) incl += up;
        }
        if (b < a.B) rt_first[b] = carry + incl - ch;
        carry += __shfl(incl, kWave - 1);
      }
      if (lane == 0) rt_total = carry;
    }
    __syncthreads();
    Nc = rt_total;
    Pw = Nc < a.P ? (Nc > 0 ? Nc : 1) : a.P;
    if (blockIdx.x == 0) {
      for (int b = tid; b < a.B; b += kDecodeThreads) a.ws_rowinfo[b * 4 + 3] = rt_first[b];
      if (tid == 0) {
        a.ws_hdr[0] = Nc;
        a.ws_hdr[1] = Pw;
      }
    }
  } else {
    Nc = a.ws_hdr[0];
    Pw = a.ws_hdr[1];
  }
  const int64_t w = blockIdx.x * static_cast<int64_t>(kDecodeWaves) + wave;
  if (w >= Pw) return;
  const int32_t lead = effective_lead(Nc, Pw, a.lead);
  const int64_t x_begin = worker_start(w, Nc, Pw, lead), x_end = worker_start(w + 1, Nc, Pw, lead);
  if (x_begin >= x_end) return;

  ChunkPos pos;
  if (fused) {
    int lo = 0, hi = static_cast<int>(a.B) - 1;  // last row whose first chunk <= x_begin
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (rt_first[mid] <= x_begin) lo = mid; else hi = mid - 1;
    }
    const int nc = static_cast<int>(stream_chunks(rt_len[lo], rt_n[lo], C));
    const int64_t rel = x_begin - rt_first[lo];
    pos.b = lo;
    pos.kvh = static_cast<int>(rel / nc);
    pos.c = static_cast<int>(rel % nc);
  } else {
    const int4 st = *reinterpret_cast<const int4*>(wstart + w * 4);
    pos.b = st.x;
    pos.kvh = st.y;
    pos.c = st.z;
  }
  pos.len = row_len(pos.b);
  pos.n = row_n(pos.b);
  pos.nc = static_cast<int>(stream_chunks(pos.len, pos.n, C));

  const uint8_t* kin = static_cast<const uint8_t*>(a.kc_in);
  const uint8_t* vin = static_cast<const uint8_t*>(a.vc_in);
  const T* qv = static_cast<const T*>(a.query);
  T* att = static_cast<T*>(a.attention);

  float o_acc[ROWS][DV];  // this lane's slot's share of each row's context
  Acc seg_m[ROWS], seg_l[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    seg_m[r] = neg_inf;
    seg_l[r] = 0;
#pragma unroll
    for (int i = 0; i < DV; i++) o_acc[r][i] = 0.0f;
  }

  for (int64_t x = x_begin; x < x_end; x++) {
    const int64_t grp = static_cast<int64_t>(pos.b) * Hk + pos.kvh;
    const bool is_new = pos.c == pos.nc - 1;  // the last chunk holds the appended rows
    const int j0 = is_new ? pos.len : pos.c * C;
    const int n_all = is_new ? pos.n : (pos.c * C + C < pos.len ? C : pos.len - pos.c * C);
    // the chunk's rows: cached ones from the cache (dense or through the
    // block table: a chunk lies inside one block), appended ones from the new
    // rows; a table entry outside the pool reads as zero rows
    const uint8_t* krows = kin;
    const uint8_t* vrows = vin;
    uint32_t kbytes = static_cast<uint32_t>(n_all) * KROW, vbytes = static_cast<uint32_t>(n_all) * VROW;
    if (is_new) {
      krows = static_cast<const uint8_t*>(a.new_key) + grp * Q * KROW;
      vrows = static_cast<const uint8_t*>(a.new_value) + grp * Q * VROW;
    } else if (a.paged) {
      const uint8_t* k0 = slot_row(a, kin, pos.b, pos.kvh, static_cast<int64_t>(pos.c) * C, KROW);
      const uint8_t* v0 = slot_row(a, vin, pos.b, pos.kvh, static_cast<int64_t>(pos.c) * C, VROW);
      krows = k0 ? k0 : kin;
      vrows = v0 ? v0 : vin;
      kbytes = k0 ? kbytes : 0u;
      vbytes = v0 ? vbytes : 0u;
    } else {
      krows = kin + (grp * M + pos.c * C) * KROW;
      vrows = vin + (grp * M + pos.c * C) * VROW;
    }
    uint4 kx[NK], vx[NV];
    {
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(krows, kbytes);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vrows, vbytes);
#pragma unroll
      for (int i = 0; i < NK; i++)
        kx[i] = buf_ld16<kNonTemporal>(rk, static_cast<uint32_t>(lane * KROW + 16 * i));
#pragma unroll
      for (int i = 0; i < NV; i++)
        vx[i] = buf_ld16<kNonTemporal>(rv, static_cast<uint32_t>(lane * VROW + 16 * i));
    }
    if (a.out_of_place) {  // every visited slot goes to the output cache
      const __amdgpu_buffer_rsrc_t wk =
          make_rsrc(static_cast<uint8_t*>(a.kc_out) + (grp * M + j0) * KROW, static_cast<uint32_t>(n_all) * KROW);
      const __amdgpu_buffer_rsrc_t wv =
          make_rsrc(static_cast<uint8_t*>(a.vc_out) + (grp * M + j0) * VROW, static_cast<uint32_t>(n_all) * VROW);
#pragma unroll
      for (int i = 0; i < NK; i++) buf_st16(wk, static_cast<uint32_t>(lane * KROW + 16 * i), kx[i]);
#pragma unroll
      for (int i = 0; i < NV; i++) buf_st16(wv, static_cast<uint32_t>(lane * VROW + 16 * i), vx[i]);
    }

    // ---- scores of this lane's slot for every packed row ----
    Acc s[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const int t = r % Q, g = r / Q;
      const bool row_ok = r < R && t < pos.n;
      const int64_t qrow = (static_cast<int64_t>(pos.b) * a.Hq + pos.kvh * a.G + g) * Q + t;
      Acc dot = 0;
      if (row_ok) {
#pragma unroll
        for (int i = 0; i < NK; i++)
          dot += Mth::dot(*reinterpret_cast<const uint4*>(qv + qrow * D + i * (16 / sizeof(T))),
                          kx[i]);
      }
      const bool ok = row_ok && lane < n_all && j0 + lane <= pos.len + t;
      s[r] = ok ? dot * scale : neg_inf;
    }

    // ---- chunk statistics per row, attention values, segment update ----
    float pb[ROWS];  // p * beta: this slot's context weight per row
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const int t = r % Q, g = r / Q;
      const bool row_ok = r < R && t < pos.n;
      const Acc m_c = small_reduce<true>(s[r]);
      const Acc p = s[r] == neg_inf ? Acc(0) : acc_exp(s[r] - m_c);
      const Acc l_c = small_reduce<false>(p);
      const Acc m_new = m_c > seg_m[r] ? m_c : seg_m[r];
      const Acc alpha = seg_m[r] == neg_inf ? Acc(0) : acc_exp(seg_m[r] - m_new);
      const Acc beta = m_c == neg_inf ? Acc(0) : acc_exp(m_c - m_new);
      seg_l[r] = seg_l[r] * alpha + l_c * beta;
      seg_m[r] = m_new;
      pb[r] = static_cast<float>(p * beta);
      const float al = static_cast<float>(alpha);
#pragma unroll
      for (int i = 0; i < DV; i++) o_acc[r][i] *= al;
      if (row_ok) {
        if (lane == 0) {
          double* cm = a.ws_chunk_ml + ((grp * a.nchunk_max + pos.c) * R + r) * 2;
          cm[0] = static_cast<double>(m_c);
          cm[1] = static_cast<double>(l_c);
        }
        if (lane < n_all && !a.read_only) {
          const int64_t arow = (static_cast<int64_t>(pos.b) * a.Hq + pos.kvh * a.G + g) * Q + t;
          E::store(att + arow * M + j0 + lane, p);
        }
      }
    }
    // ---- context: this lane's slot's V row weighted per row ----
#pragma unroll
    for (int i = 0; i < NV; i++) {
      float v[16 / sizeof(T)];
      if constexpr (sizeof(T) == 2) {
        const uint32_t wv[4] = {vx[i].x, vx[i].y, vx[i].z, vx[i].w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          v[2 * e] = __uint_as_float(wv[e] << 16);
          v[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
        }
      } else {
        v[0] = __uint_as_float(vx[i].x);
        v[1] = __uint_as_float(vx[i].y);
        v[2] = __uint_as_float(vx[i].z);
        v[3] = __uint_as_float(vx[i].w);
      }
#pragma unroll
      for (int r = 0; r < ROWS; r++)
#pragma unroll
        for (int e = 0; e < static_cast<int>(16 / sizeof(T)); e++)
          o_acc[r][i * (16 / sizeof(T)) + e] += pb[r] * v[e];
    }

    // ---- the next chunk's position ----
    ChunkPos nxt = pos;
    bool group_ends = false;
    nxt.c++;
    if (nxt.c == nxt.nc) {
      group_ends = true;
      nxt.c = 0;
      nxt.kvh++;
      if (nxt.kvh == Hk) {
        nxt.kvh = 0;
        do {
          nxt.b++;
          if (nxt.b >= a.B) break;
          nxt.len = row_len(nxt.b);
          nxt.n = row_n(nxt.b);
          nxt.nc = static_cast<int>(stream_chunks(nxt.len, nxt.n, C));
        } while (nxt.nc == 0);
      }
    }

    // ---- flush the segment when the KV head changes or at the end ----
    if (group_ends || x + 1 == x_end) {
      const int64_t seg = w + grp;
      // the rows' contexts summed over the wave's slots, scattered over the
      // lanes (value r * DV + i is row r, dim i)
      constexpr int NO = ROWS * DV;
      float flat[NO];
#pragma unroll
      for (int r = 0; r < ROWS; r++)
#pragma unroll
        for (int i = 0; i < DV; i++) {
          flat[r * DV + i] = o_acc[r][i];
          o_acc[r][i] = 0.0f;
        }
      sum_scatter<NO>(flat, lane);
      constexpr int PER = NO >= kWave ? NO / kWave : 1;  // values a lane holds
      constexpr int SHARE = NO >= kWave ? 1 : kWave / NO;  // lanes per value
#pragma unroll
      for (int k = 0; k < PER; k++) {
        const int idx = NO >= kWave ? lane * PER + k : lane / SHARE;
        const int r = idx / DV, i = idx % DV;
        if (r < R && lane % SHARE == 0) a.ws_seg_o[(seg * R + r) * DV + i] = flat[k];
      }
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        if (r < R && lane == 0) {
          double* ml = a.ws_seg_ml + (seg * R + r) * 2;
          ml[0] = static_cast<double>(seg_m[r]);
          ml[1] = static_cast<double>(seg_l[r]);
        }
        seg_m[r] = neg_inf;
        seg_l[r] = 0;
      }
    }
    pos = nxt;
  }
}

}  // namespace kvc
