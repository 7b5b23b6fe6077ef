// kvc_decode.h -- stream-mode attend kernel for decode-shaped steps: the
// packed query rows of one KV head (Hq/Hk query heads x Q tokens) are few
// (<= 8), so the step is a stream over the visible K/V prefix with ~4
// flop/byte; it is bound by HBM bandwidth, not by arithmetic.
//
// Work split ("stream-K" over cache slots, per wave): the visible slots of
// every (batch row, KV head) are cut into chunks of C slots; the flattened
// chunk list (row-major over b, head, chunk) is divided into equal
// contiguous ranges, one per wave of the grid, so ragged lengths cost no
// imbalance and no wave waits for another (there is no workgroup barrier).
// A wave keeps running softmax statistics across the chunks of one KV head
// (a "segment") and writes one partial per segment; the combine kernel
// merges them.
//
// Per chunk a wave
//   - issues its 16-byte K loads (lane l reads dims [(l % LK)*VEC, +VEC) of
//     slot l / LK of every 1 KB load, so each load instruction reads
//     contiguous bytes), computes partial dot products for all packed rows
//     and reduces them across the LK lanes of a slot with a butterfly
//     reduce-scatter (each lane ends with whole dot products);
//   - takes per-row chunk statistics m_c, l_c over its LDS score tile,
//     writes exp(s - m_c) to the attention buffer and (m_c, l_c) to the
//     workspace, and folds the chunk into its running segment statistics;
//   - issues its V loads into the registers K used and accumulates the
//     context partial o += p * v.
// The same loads feed the cache writes: out of place every visited slot is
// stored to the output cache (the copy the page's contract requires), in
// place only the appended rows are stored.
//
// The step follows "Autoregressive KV-cache append and causal attention",
// Required behavior: KV head floor(h / (Hq/Hk)) per query head, slot
// length + t for appended row t, visibility j <= length + t (lower-right
// alignment, KempnerForge PR 542, Summary), scores scale * dot(q, k) and a
// max-subtracted softmax.
#pragma once

#include "kvc_common.h"

namespace kvc {

constexpr int kDecodeThreads = 256;
constexpr int kDecodeWaves = kDecodeThreads / kWave;

// ---- element-type specific pieces ------------------------------------------
template <typename T>
struct DecodeMath;

template <>
struct DecodeMath<bf16> {
  static constexpr int kVec = 8;  // elements per 16 bytes
  using Acc = float;
  // sum_i q_i k_i over 8 bf16 pairs with fp32 accumulation (v_dot2 bf16)
  __device__ __forceinline__ static float dot(const uint4& q, const uint4& k) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float acc = 0.0f;
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x),
                                          __builtin_bit_cast(bf16x2, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y),
                                          __builtin_bit_cast(bf16x2, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z),
                                          __builtin_bit_cast(bf16x2, k.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w),
                                          __builtin_bit_cast(bf16x2, k.w), acc, false);
    return acc;
  }
  // o[i] += p * v_i for the 8 bf16 values of v
  __device__ __forceinline__ static void axpy(float p, const uint4& v, float (&o)[kVec]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      o[2 * i] += p * __uint_as_float(w[i] << 16);
      o[2 * i + 1] += p * __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

template <>
struct DecodeMath<float> {
  static constexpr int kVec = 4;
  using Acc = double;  // fp32 scores reach ~1e3; keep them exact to 1e-5
  __device__ __forceinline__ static double dot(const uint4& q, const uint4& k) {
    double acc = static_cast<double>(__uint_as_float(q.x)) * __uint_as_float(k.x);
    acc += static_cast<double>(__uint_as_float(q.y)) * __uint_as_float(k.y);
    acc += static_cast<double>(__uint_as_float(q.z)) * __uint_as_float(k.z);
    acc += static_cast<double>(__uint_as_float(q.w)) * __uint_as_float(k.w);
    return acc;
  }
  __device__ __forceinline__ static void axpy(float p, const uint4& v, float (&o)[kVec]) {
    o[0] += p * __uint_as_float(v.x);
    o[1] += p * __uint_as_float(v.y);
    o[2] += p * __uint_as_float(v.z);
    o[3] += p * __uint_as_float(v.w);
  }
};

// Butterfly reduce-scatter over the W lanes that share one slot: lane kc
// (its index within the W lanes) starts with N partial sums and ends with
// the complete sums of entries [kc * N / W, (kc + 1) * N / W) in v[0 ..).
template <int W, int LEN, typename A, int N>
__device__ __forceinline__ void reduce_scatter(A (&v)[N], int kc) {
  if constexpr (W >= 1 && LEN >= 2) {
    const bool upper = (kc & W) != 0;
#pragma unroll
    for (int i = 0; i < LEN / 2; i++) {
      const A lo = v[i], hi = v[i + LEN / 2];
      const A send = upper ? lo : hi;
      const A keep = upper ? hi : lo;
      v[i] = keep + __shfl_xor(send, W);
    }
    reduce_scatter<W / 2, LEN / 2>(v, kc);
  }
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *static_cast<const uint4*>(p); }

// Raw buffer access (gfx9 MUBUF): a descriptor holds a base address and a
// byte count; a 16-byte load whose offset is >= the count returns zeros and
// such a store is dropped.  Offsets are unsigned 32-bit, so an offset
// computed as a negative number is out of range too.  The chunk bounds of
// the decode kernel are expressed this way instead of with branches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferDword3 = 0x00020000;  // gfx9: 32-bit data format, raw access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufferDword3);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, static_cast<int>(off), 0, 0);
}

// Chunk size for a (D, Dv) pair: one wave's chunk is at most 16 loads of
// 16 bytes per lane for K and for V, and at most 64 slots (one per lane in
// the statistics step).
template <typename T, int D, int DV>
constexpr int decode_chunk() {
  constexpr int E = sizeof(T);
  constexpr int spl_k = kWave / (D * E / 16), spl_v = kWave / (DV * E / 16);
  constexpr int spl = spl_k < spl_v ? spl_k : spl_v;
  return 16 * spl < kWave ? 16 * spl : kWave;
}

// Wave-local ordering of LDS accesses (all lanes of one wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// One chunk of one cache tensor (K or V, rows of ROWB bytes) for one wave:
// loads slot jl = u * SPL + lane_slot into buf[u] (cached rows [0, n_old)
// from the cache, appended rows [n_old, n_all) from the new rows), and
// writes the visited rows to the output cache (all of them out of place,
// the appended ones in place).
template <int U, int SPL, int ROWB>
__device__ __forceinline__ void chunk_rows(uint4 (&buf)[16], const uint8_t* cache_in,
                                           uint8_t* cache_out, const uint8_t* new_rows,
                                           uint32_t lane_off, int n_old, int n_all, bool oop) {
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(cache_in, static_cast<uint32_t>(n_old) * ROWB);
#pragma unroll
  for (int u = 0; u < U; u++) buf[u] = buf_ld16(rc, lane_off + u * SPL * ROWB);
  const uint32_t shift = static_cast<uint32_t>(n_old) * ROWB;  // appended rows start here
  if (n_old < n_all) {
    const __amdgpu_buffer_rsrc_t rn =
        make_rsrc(new_rows, static_cast<uint32_t>(n_all - n_old) * ROWB);
#pragma unroll
    for (int u = 0; u < U; u++) {
      const uint4 x = buf_ld16(rn, lane_off + u * SPL * ROWB - shift);
      buf[u].x |= x.x;
      buf[u].y |= x.y;
      buf[u].z |= x.z;
      buf[u].w |= x.w;
    }
  }
  if (oop) {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(cache_out, static_cast<uint32_t>(n_all) * ROWB);
#pragma unroll
    for (int u = 0; u < U; u++) buf_st16(ro, lane_off + u * SPL * ROWB, buf[u]);
  } else if (n_old < n_all) {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(cache_out + shift,
                                                static_cast<uint32_t>(n_all - n_old) * ROWB);
#pragma unroll
    for (int u = 0; u < U; u++) buf_st16(ro, lane_off + u * SPL * ROWB - shift, buf[u]);
  }
}

template <typename T, int D, int DV, int ROWS, bool Q1>
__global__ __launch_bounds__(kDecodeThreads) void attend_decode_kernel(StepArgs a) {
  using Mth = DecodeMath<T>;
  using Acc = typename Mth::Acc;
  constexpr int E = sizeof(T);
  constexpr int VEC = Mth::kVec;
  constexpr int LK = D * E / 16, SPLK = kWave / LK;   // lanes per K row, K rows per load
  constexpr int LV = DV * E / 16, SPLV = kWave / LV;  // same for V
  constexpr int C = decode_chunk<T, D, DV>();         // slots per chunk (one wave)
  constexpr int UK = C / SPLK, UV = C / SPLV;         // 16-byte loads per lane
  constexpr int GU = LK / ROWS > 1 ? LK / ROWS : 1;   // loads per reduce-scatter group
  constexpr int NV = GU * ROWS;                       // partial dots per group
  constexpr int KPL = NV / LK;                        // finished dots per lane
  constexpr int KROW = D * E, VROW = DV * E;          // row bytes
  static_assert(D * E % 16 == 0 && DV * E % 16 == 0 && LK <= kWave && LV <= kWave, "head size");
  static_assert(UK >= 1 && UK <= 16 && UV >= 1 && UV <= 16 && UK % GU == 0, "chunk shape");
  static_assert(NV % LK == 0 && KPL >= 1 && C <= kWave, "row shape");

  __shared__ Acc sc_all[kDecodeWaves][ROWS][C];

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  Acc (*sc)[C] = sc_all[wave];
  const int ks = lane / LK, kc = lane % LK;
  const int vs = lane / LV, vc = lane % LV;
  const uint32_t k_off = static_cast<uint32_t>(ks * KROW + kc * 16);
  const uint32_t v_off = static_cast<uint32_t>(vs * VROW + vc * 16);
  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  const Acc scale = static_cast<Acc>(a.scale);
  const int Q = Q1 ? 1 : static_cast<int>(a.Q);
  const int R = static_cast<int>(a.R);
  const int Hk = static_cast<int>(a.Hk);
  const int64_t M = a.M;

  const int64_t Nc = a.ws_hdr[0];
  const int64_t Pw = a.P;  // stream workers = waves of the grid
  const int64_t w = blockIdx.x * static_cast<int64_t>(kDecodeWaves) + wave;
  const int64_t x_begin = w * Nc / Pw, x_end = (w + 1) * Nc / Pw;
  if (x_begin >= x_end) return;

  // locate the first chunk: the last row whose first chunk index <= x_begin
  int lo = 0, hi = static_cast<int>(a.B) - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (a.ws_rowinfo[mid * 4 + 3] <= x_begin) lo = mid; else hi = mid - 1;
  }
  int b = lo;
  int len = static_cast<int>(a.ws_rowinfo[b * 4 + 0]);
  int n = static_cast<int>(a.ws_rowinfo[b * 4 + 1]);
  int nc = static_cast<int>(row_chunks(len, n, C));
  int kvh, c;
  {
    const int rel = static_cast<int>(x_begin - a.ws_rowinfo[b * 4 + 3]);
    kvh = rel / nc;
    c = rel % nc;
  }

  const T* qbase = static_cast<const T*>(a.query);
  const uint8_t* kin = static_cast<const uint8_t*>(a.kc_in);
  const uint8_t* vin = static_cast<const uint8_t*>(a.vc_in);
  uint8_t* kout = static_cast<uint8_t*>(a.kc_out);
  uint8_t* vout = static_cast<uint8_t*>(a.vc_out);
  const uint8_t* nkb = static_cast<const uint8_t*>(a.new_key);
  const uint8_t* nvb = static_cast<const uint8_t*>(a.new_value);
  T* att = static_cast<T*>(a.attention);
  const bool oop = a.out_of_place != 0;

  uint4 qf[ROWS];
  float o_acc[ROWS][VEC];
  Acc seg_m[ROWS], seg_l[ROWS];
  bool new_group = true;
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    seg_m[r] = neg_inf;
    seg_l[r] = 0;
#pragma unroll
    for (int i = 0; i < VEC; i++) o_acc[r][i] = 0.0f;
  }

  for (int64_t x = x_begin; x < x_end; x++) {
    const int64_t grp = static_cast<int64_t>(b) * Hk + kvh;
    const int j0 = c * C;
    const int new_len = len + n;
    const int j1 = j0 + C < new_len ? j0 + C : new_len;  // chunk end
    const int n_all = j1 - j0;                           // visited slots
    const int n_old = len - j0 < 0 ? 0 : (len - j0 < n_all ? len - j0 : n_all);  // cached ones
    if (new_group) {
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        const int t = Q1 ? 0 : r % Q;
        const int g = Q1 ? r : r / Q;
        const bool valid = r < R && t < n;
        const int64_t row = (static_cast<int64_t>(b) * a.Hq + kvh * a.G + g) * Q + t;
        qf[r] = valid ? ld16(qbase + row * D + kc * VEC) : make_uint4(0, 0, 0, 0);
      }
      new_group = false;
    }

    // ---- K rows of the chunk: loads, cache writes, scores ----
    uint4 buf[16];
    chunk_rows<UK, SPLK, KROW>(buf, kin + (grp * M + j0) * KROW, kout + (grp * M + j0) * KROW,
                               nkb + (grp * a.Q + (j0 + n_old - len)) * KROW, k_off, n_old,
                               n_all, oop);
#pragma unroll
    for (int g0 = 0; g0 < UK; g0 += GU) {
      Acc part[NV];
#pragma unroll
      for (int gu = 0; gu < GU; gu++)
#pragma unroll
        for (int r = 0; r < ROWS; r++) part[gu * ROWS + r] = Mth::dot(qf[r], buf[g0 + gu]);
      reduce_scatter<LK / 2, NV>(part, kc);
#pragma unroll
      for (int k = 0; k < KPL; k++) {
        const int i = kc * KPL + k;
        const int gu = i / ROWS, r = i % ROWS;
        const int jl = (g0 + gu) * SPLK + ks;
        // visible: an existing row r (< R) whose token t is appended
        // (t < n) and slot j0 + jl <= len + t
        const int t = Q1 ? 0 : r % Q;
        const bool ok = r < R && t < n && jl < n_all && j0 + jl <= len + t;
        sc[r][jl] = ok ? part[k] * scale : neg_inf;
      }
    }
    wave_lds_sync();

    // ---- chunk statistics, attention values, segment update ----
    Acc alpha[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const Acc s = lane < C ? sc[r][lane] : neg_inf;
      const Acc m = wave_max(s);
      const Acc p = s == neg_inf ? Acc(0) : acc_exp(s - m);
      const Acc l = wave_sum(p);
      const Acc m_new = m > seg_m[r] ? m : seg_m[r];
      alpha[r] = seg_m[r] == neg_inf ? Acc(0) : acc_exp(seg_m[r] - m_new);
      const Acc beta = m == neg_inf ? Acc(0) : acc_exp(m - m_new);
      seg_l[r] = seg_l[r] * alpha[r] + l * beta;
      seg_m[r] = m_new;
      const int t = Q1 ? 0 : r % Q;
      if (r < R && t < n) {
        const int g = Q1 ? r : r / Q;
        const int64_t row = (static_cast<int64_t>(b) * a.Hq + kvh * a.G + g) * Q + t;
        if (lane < n_all) Elem<T>::store(att + row * M + j0 + lane, p);
        if (lane == 0) {
          double* cm = a.ws_chunk_ml + ((grp * a.nchunk_max + c) * R + r) * 2;
          cm[0] = static_cast<double>(m);
          cm[1] = static_cast<double>(l);
        }
      }
      if (lane < C) sc[r][lane] = p * beta;
    }
    wave_lds_sync();

    // ---- V rows of the chunk (same registers), cache writes, context ----
    chunk_rows<UV, SPLV, VROW>(buf, vin + (grp * M + j0) * VROW, vout + (grp * M + j0) * VROW,
                               nvb + (grp * a.Q + (j0 + n_old - len)) * VROW, v_off, n_old,
                               n_all, oop);
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const float al = static_cast<float>(alpha[r]);
#pragma unroll
      for (int i = 0; i < VEC; i++) o_acc[r][i] *= al;
    }
#pragma unroll
    for (int u = 0; u < UV; u++) {
      const int jl = u * SPLV + vs;  // p is 0 for slots past the chunk end
#pragma unroll
      for (int r = 0; r < ROWS; r++) Mth::axpy(static_cast<float>(sc[r][jl]), buf[u], o_acc[r]);
    }
    wave_lds_sync();  // the next chunk overwrites the tile

    // ---- advance; flush the segment when the KV head changes or at the end ----
    const int64_t prev_grp = grp;
    c++;
    if (c == nc) {
      c = 0;
      kvh++;
      new_group = true;
      if (kvh == Hk) {
        kvh = 0;
        do {
          b++;
          if (b >= a.B) break;
          len = static_cast<int>(a.ws_rowinfo[b * 4 + 0]);
          n = static_cast<int>(a.ws_rowinfo[b * 4 + 1]);
          nc = static_cast<int>(row_chunks(len, n, C));
        } while (nc == 0);
      }
    }
    if (new_group || x + 1 == x_end) {
      // sum o over the lanes that hold the same dims
#pragma unroll
      for (int off = LV; off < kWave; off <<= 1)
#pragma unroll
        for (int r = 0; r < ROWS; r++)
#pragma unroll
          for (int i = 0; i < VEC; i++) o_acc[r][i] += __shfl_xor(o_acc[r][i], off);
      const int64_t seg = w + prev_grp;
      if (vs == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
          if (r < R) {
            float* dst = a.ws_seg_o + (seg * R + r) * DV + vc * VEC;
#pragma unroll
            for (int i = 0; i < VEC; i++) dst[i] = o_acc[r][i];
          }
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
          if (r < R) {
            double* ml = a.ws_seg_ml + (seg * R + r) * 2;
            ml[0] = static_cast<double>(seg_m[r]);
            ml[1] = static_cast<double>(seg_l[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        seg_m[r] = neg_inf;
        seg_l[r] = 0;
#pragma unroll
        for (int i = 0; i < VEC; i++) o_acc[r][i] = 0.0f;
      }
    }
  }
}

}  // namespace kvc
