// kvc_decode.h -- stream-mode attend kernel for decode-shaped steps: the
// packed query rows of one KV head (Hq/Hk query heads x Q tokens) are few
// (<= 8), so the step is a stream over the visible K/V prefix with ~4
// flop/byte; it is bound by HBM bandwidth, not by arithmetic.
//
// Work split ("stream-K" over cache slots, per wave): the visible slots of
// every (batch row, KV head) are cut into chunks of C slots; the flattened
// chunk list (row-major over b, head, chunk) is divided into equal
// contiguous ranges, one per wave, so ragged lengths cost no imbalance and
// no wave waits for another (there is no workgroup barrier).  A wave keeps
// running softmax statistics across the chunks of one KV head (a
// "segment") and writes one partial per segment; the combine kernel merges
// them.
//
// Per chunk a wave
//   - receives its K rows (16-byte loads issued one chunk ahead: lane l
//     holds dims [(l % LK)*VEC, +VEC) of slot l / LK of every 1 KB load, so
//     each load instruction reads contiguous bytes) and its V rows (issued
//     before the chunk's K math), so loads stay in flight during compute;
//   - computes partial dot products for every packed row and finishes them
//     with a butterfly reduce-scatter across the LK lanes of a slot (DPP
//     lane exchanges); lane (ks, kc) ends with the score of row kc % ROWS;
//   - takes per-row chunk statistics m_c, l_c (DPP rotations inside each
//     16-lane row, then lane reads across rows), writes exp(s - m_c) to the
//     attention buffer and (m_c, l_c) to the workspace, and folds the chunk
//     into its running segment statistics;
//   - accumulates the context partial o += p * v (bf16: p rounded to bf16,
//     two slots per v_dot2; fp32: fp32 FMAs).
// The chunks of a (batch row, KV head) are its cached slots in chunks of C
// and one last chunk with the appended rows, read from new_key/new_value
// (stream_chunks).  Out of place the same loads feed the cache copy the
// page's contract requires (every visited slot is stored to the output
// cache); in place the appended rows are stored by the combine kernel,
// which runs after this one.  So no kernel has to run before this one: for
// batches of up to kDecodeFusedRows rows each workgroup also works out the
// row information itself (FUSED).
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

// ---- lane exchange -----------------------------------------------------------
// DPP controls (gfx9): quad permutations, 16-lane row mirror / half mirror
// and row rotations.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i inside each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i inside each 16
constexpr int dpp_row_ror(int n) { return 0x120 + n; }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const int2 w = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __builtin_amdgcn_update_dpp(0, w.x, CTRL, 0xF, 0xF, false);
  r.y = __builtin_amdgcn_update_dpp(0, w.y, CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ float lane_read(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ double lane_read(double v, int lane) {
  const int2 w = __builtin_bit_cast(int2, v);
  int2 r;
  r.x = __builtin_amdgcn_readlane(w.x, lane);
  r.y = __builtin_amdgcn_readlane(w.y, lane);
  return __builtin_bit_cast(double, r);
}

// Value held by the lane paired with this one at butterfly step W (an
// involution that pairs the two W-halves of every 2W-lane group).
template <int W, typename A>
__device__ __forceinline__ A partner(A v) {
  if constexpr (W == 1) return dpp<kDppXor1>(v);
  else if constexpr (W == 2) return dpp<kDppXor2>(v);
  else if constexpr (W == 4) return dpp<kDppHalfMirror>(v);
  else if constexpr (W == 8) return dpp<kDppMirror>(v);
  else return __shfl_xor(v, W);
}

// Butterfly reduce-scatter over the W lanes that share one slot: lane kc
// (its index within those lanes) starts with N partial sums and ends with
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
      v[i] = keep + partner<W>(send);
    }
    reduce_scatter<W / 2, LEN / 2>(v, kc);
  }
}

// Reduce (max or sum) over the lanes of each 16-lane row that are
// congruent modulo S0 (rotations by S0, 2*S0, ..., 8).
template <int S, bool MAX, typename A>
__device__ __forceinline__ A rot_reduce(A v) {
  if constexpr (S < 16) {
    const A w = dpp<dpp_row_ror(S)>(v);
    v = MAX ? (v > w ? v : w) : v + w;
    return rot_reduce<2 * S, MAX>(v);
  } else {
    return v;
  }
}

// Per-row results: lane r (r < ROWS) of every 16-lane row holds that row's
// partial for packed row r after rot_reduce<ROWS>; combine the four rows.
template <int ROWS, bool MAX, typename A>
__device__ __forceinline__ void rows_finish(A v, A (&out)[ROWS]) {
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    A x = lane_read(v, r);
#pragma unroll
    for (int k = 1; k < kWave / 16; k++) {
      const A y = lane_read(v, 16 * k + r);
      x = MAX ? (x > y ? x : y) : x + y;
    }
    out[r] = x;
  }
}

// ---- element-type specific pieces ------------------------------------------
template <typename T>
struct DecodeMath;

template <>
struct DecodeMath<bf16> {
  static constexpr int kVec = 8;  // elements per 16 bytes
  using Acc = float;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  __device__ __forceinline__ static float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
  // sum_i q_i k_i over 8 bf16 pairs with fp32 accumulation (v_dot2 bf16)
  __device__ __forceinline__ static float dot(const uint4& q, const uint4& k) {
    float acc = dot2(q.x, k.x, 0.0f);
    acc = dot2(q.y, k.y, acc);
    acc = dot2(q.z, k.z, acc);
    acc = dot2(q.w, k.w, acc);
    return acc;
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
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *static_cast<const uint4*>(p); }

// Raw buffer access (gfx9 MUBUF): a descriptor holds a base address and a
// byte count; a 16-byte load whose offset is >= the count returns zeros and
// such a store is dropped.  Offsets are unsigned 32-bit, so an offset
// computed as a negative number is out of range too.  The chunk bounds of
// the decode kernel are expressed this way instead of with branches.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferDword3 = 0x00020000;  // gfx9: 32-bit data format, raw access

// Every descriptor here is built from wave-uniform values; reading them
// through readfirstlane keeps the descriptor in scalar registers (a
// descriptor the compiler places in vector registers costs a loop per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* q = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, static_cast<short>(0), static_cast<int>(n),
                                           kBufferDword3);
}
// Cache policy operand of a buffer load: 0 (default) or kNonTemporal (the
// nt bit), for data read once, which then does not allocate in the caches
// as if it were going to be read again.
constexpr int kNonTemporal = 2;
template <int POLICY = 0>
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, POLICY);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Non-temporal store (the copy into the output cache, not read again by the step).
__device__ __forceinline__ void buf_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, static_cast<int>(off), 0, kNonTemporal);
}

// Chunk size: one wave's chunk is at most 64 slots and at most 16 loads of
// 16 bytes per lane for K and for V (8 when fp32 scores need the
// registers), since both tensors' loads are in flight at once.
template <typename T, int D, int DV, int ROWS>
constexpr int decode_chunk() {
  constexpr int E = sizeof(T);
  constexpr int spl_k = kWave / (D * E / 16), spl_v = kWave / (DV * E / 16);
  constexpr int spl = spl_k < spl_v ? spl_k : spl_v;
  constexpr int loads = E == 4 ? 8 : 16;
  return loads * spl < kWave ? loads * spl : kWave;
}

// Resident waves per SIMD the decode kernel is built for: 8 packed rows
// (their context accumulators and query rows) need a SIMD's whole register
// file; the grid then holds one workgroup per compute unit.
template <int ROWS>
constexpr int decode_waves_per_simd() {
  return ROWS > 4 ? 1 : 2;
}

// Wave-local ordering of LDS accesses (all lanes of one wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The rows of one tensor a chunk visits: `bytes` bytes of rows at `rows`.
// A zero count makes every load return zeros.
struct RowSrc {
  const uint8_t* rows;
  uint32_t bytes;
};

// The 16-byte load u of a chunk (slot u * rows-per-load + lane slot; one
// load covers 1 KB): the descriptor is rebased every 4 loads so that the
// lane offset plus an immediate below 4 KB addresses the whole group.
// Every K/V row is read once per step, so the loads are non-temporal
// (with the default policy the kernel takes ~16 % longer at 32 sequences
// of up to 8192 slots: the caches fill with rows nobody reads again).
__device__ __forceinline__ uint4 load_one(const RowSrc& s, int u, uint32_t lane_off) {
  const uint32_t base = static_cast<uint32_t>(u / 4) * 4096u;
  const uint32_t imm = static_cast<uint32_t>(u % 4) * 1024u;
  const uint32_t left = s.bytes > base ? s.bytes - base : 0u;
  return buf_ld16<kNonTemporal>(make_rsrc(s.rows + base, left), lane_off + imm);
}

// Out of place: the copy of the visited rows to the output cache (load u of
// the chunk, same addressing as load_one; `bytes` = 0 stores nothing).
__device__ __forceinline__ void store_one(uint8_t* out, uint32_t bytes, int u,
                                          uint32_t lane_off, const uint4& v) {
  const uint32_t base = static_cast<uint32_t>(u / 4) * 4096u;
  const uint32_t imm = static_cast<uint32_t>(u % 4) * 1024u;
  const uint32_t left = bytes > base ? bytes - base : 0u;
  buf_st16(make_rsrc(out + base, left), lane_off + imm, v);
}

// Batches of up to this many rows are prepared by the decode kernel itself
// (a row table in LDS); larger ones by the prep kernel.
constexpr int kDecodeFusedRows = 1024;

// Position of a wave in the flattened chunk list (all fields wave-uniform).
struct ChunkPos {
  int b, kvh, c;   // batch row, KV head, chunk within the head
  int len, n, nc;  // the row's old length, appended rows, chunks per head
};

template <typename T, int D, int DV, int ROWS, bool Q1, bool OOP, bool FUSED, bool PAGED>
__global__ __launch_bounds__(kDecodeThreads)
__attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<ROWS>()))) void attend_decode_kernel(
    StepArgs a, const int64_t* __restrict__ rowinfo, const int32_t* __restrict__ wstart) {
  using Mth = DecodeMath<T>;
  using Acc = typename Mth::Acc;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int E = sizeof(T);
  constexpr int VEC = Mth::kVec;
  constexpr int LK = D * E / 16, SPLK = kWave / LK;   // lanes per K row, K rows per load
  constexpr int LV = DV * E / 16, SPLV = kWave / LV;  // same for V
  constexpr int C = decode_chunk<T, D, DV, ROWS>();   // slots per chunk (one wave)
  constexpr int UK = C / SPLK, UV = C / SPLV;         // 16-byte loads per lane
  constexpr int GU = LK / ROWS;                       // loads per reduce-scatter group
  constexpr int NG = UK / GU;                         // reduce-scatter groups per chunk
  constexpr int KROW = D * E, VROW = DV * E;          // row bytes
  static_assert(D * E % 16 == 0 && DV * E % 16 == 0 && LK <= kWave && LV <= kWave, "head size");
  static_assert(LK >= ROWS && LK % ROWS == 0 && ROWS < 16, "one finished dot product per lane");
  static_assert(UK >= 1 && UK <= 16 && UV >= 1 && UV <= 16 && UK % GU == 0, "chunk shape");
  static_assert(!kBf16 || (D == DV && UV % 2 == 0), "bf16 context pairs slots of equal layout");
  static_assert(SPLK * KROW == 1024 && SPLV * VROW == 1024, "one load covers 1 KB");
  static_assert((C & (C - 1)) == 0, "chunk sizes are powers of two (the combine shifts by log2 C)");
  static_assert(!(PAGED && OOP), "the paged cache is updated in place");

  // probabilities for the context step: bf16 pairs [slot pair][slot lane][row]
  // (packed bf16x2), or fp32 [row][slot]
  constexpr int PTILE = kBf16 ? (UV / 2) * SPLV * ROWS : ROWS * C;
  __shared__ uint32_t ptile_all[kDecodeWaves][PTILE];
  // exp(s - m_c) of the chunk, [row][slot], so that the attention rows leave
  // in 16-byte pieces (whole 128-byte lines when the chunk is 128 bytes)
  constexpr int AVEC = 16 / E;  // elements per 16 bytes
  static_assert(C % AVEC == 0, "attention pieces");
  __shared__ __align__(16) T atile_all[kDecodeWaves][ROWS * C];
  // FUSED: every batch row's old length, appended count and first chunk
  constexpr int RT = FUSED ? kDecodeFusedRows : 1;
  __shared__ int32_t rt_len[RT], rt_n[RT];
  __shared__ int64_t rt_first[RT];
  __shared__ int64_t rt_total;

  const int tid = threadIdx.x, lane = tid % kWave;
  // the wave index is uniform across the wave; saying so keeps everything
  // derived from it (chunk range, rows, buffer descriptors) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  uint32_t* ptile = ptile_all[wave];
  T* atile = atile_all[wave];
  const int ks = lane / LK, kc = lane % LK;
  const int vs = lane / LV, vc = lane % LV;
  const int my_row = kc % ROWS;  // packed row whose scores this lane finishes
  const uint32_t k_off = static_cast<uint32_t>(ks * KROW + kc * 16);
  const uint32_t v_off = static_cast<uint32_t>(vs * VROW + vc * 16);
  const Acc neg_inf = -static_cast<Acc>(INFINITY);
  const Acc scale = static_cast<Acc>(a.scale);
  const int Q = Q1 ? 1 : static_cast<int>(a.Q);
  const int R = static_cast<int>(a.R);
  const int Hk = static_cast<int>(a.Hk);
  const int64_t M = a.M;

  // Row information.  FUSED: the workgroup builds the table of every batch
  // row (the prep kernel's checks, each row's first chunk in the flattened
  // list) in LDS, and workgroup 0 publishes it for the combine kernel;
  // otherwise the prep kernel has written it and every worker's start.
  // hdr: [0] total chunks Nc, [1] busy stream workers Pe = min(P, Nc).
  auto row_len = [&](int b) { return FUSED ? rt_len[b] : static_cast<int>(rowinfo[b * 4 + 0]); };
  auto row_n = [&](int b) { return FUSED ? rt_n[b] : static_cast<int>(rowinfo[b * 4 + 1]); };
  int64_t Nc, Pw;
  if constexpr (FUSED) {
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
  if (x_begin >= x_end) return;  // no chunks at all (Nc = 0)

  // first chunk of this worker
  ChunkPos pos;
  if constexpr (FUSED) {
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

  const uint8_t* qbase = static_cast<const uint8_t*>(a.query);
  const uint8_t* kin = static_cast<const uint8_t*>(a.kc_in);
  const uint8_t* vin = static_cast<const uint8_t*>(a.vc_in);
  uint8_t* kout = static_cast<uint8_t*>(a.kc_out);
  uint8_t* vout = static_cast<uint8_t*>(a.vc_out);
  T* att = static_cast<T*>(a.attention);

  auto grp_of = [&](const ChunkPos& p) { return static_cast<int64_t>(p.b) * Hk + p.kvh; };
  // the last chunk of a head holds its appended rows, the others cached ones
  auto is_new_of = [&](const ChunkPos& p) { return p.c == p.nc - 1; };
  auto j0_of = [&](const ChunkPos& p) { return is_new_of(p) ? p.len : p.c * C; };
  auto n_all_of = [&](const ChunkPos& p) {
    return is_new_of(p) ? p.n : (p.c * C + C < p.len ? C : p.len - p.c * C);
  };
  // The rows a chunk visits: cached rows from the input cache, appended rows
  // from new_key / new_value (row t of the head's new rows is slot len + t).
  // live = false (past the last chunk): zero rows, so every path through
  // the loop issues the same loads.
  // Paged: a chunk lies inside one block (blocks hold a power of two >= C
  // slots), so its rows are contiguous too; an entry outside the pool reads
  // as zero rows.  FUSED: the wave keeps the blocks of its next 64 chunks
  // in LDS (entry i: chunk blk_base + i, read once per 64 chunks, so no
  // chunk waits on the table); otherwise each chunk reads its table entry.
  __shared__ int32_t blk_all[(PAGED && FUSED) ? kDecodeWaves : 1][kWave];
  int64_t blk_base = x_begin;
  auto fill_blocks = [&](int64_t x0) {
    blk_base = x0;
    if constexpr (PAGED && FUSED) {
      int32_t blk_lane = -1;
      const int64_t xl = x0 + lane;
      if (xl < x_end) {
        int lo = 0, hi = static_cast<int>(a.B) - 1;  // the row holding chunk xl
        while (lo < hi) {
          const int mid = (lo + hi + 1) / 2;
          if (rt_first[mid] <= xl) lo = mid; else hi = mid - 1;
        }
        const int nc = static_cast<int>(stream_chunks(rt_len[lo], rt_n[lo], C));
        const int rel = static_cast<int>(xl - rt_first[lo]);
        const int c = rel % nc;
        if (c != nc - 1)  // cached rows (the last chunk holds the appended ones)
          blk_lane = static_cast<int32_t>(block_of(a, lo, static_cast<int64_t>(c) * C));
      }
      blk_all[wave][lane] = blk_lane;
      wave_lds_sync();
    }
  };
  if constexpr (PAGED && FUSED) fill_blocks(x_begin);
  auto src_of = [&](const ChunkPos& p, int64_t xp, bool live, const uint8_t* cin,
                    const void* fresh, int rowb) {
    RowSrc r{cin, 0u};
    if (live) {
      const int64_t g = grp_of(p);
      r.bytes = static_cast<uint32_t>(n_all_of(p)) * rowb;
      if (is_new_of(p)) {
        r.rows = static_cast<const uint8_t*>(fresh) + g * Q * rowb;
      } else if constexpr (PAGED && FUSED) {
        const int64_t blk =
            __builtin_amdgcn_readfirstlane(blk_all[wave][static_cast<int>(xp - blk_base)]);
        const bool ok = blk >= 0 && blk < a.num_blocks;
        r.rows = cin + ((blk * Hk + p.kvh) * a.block_rows +
                        ((static_cast<int64_t>(p.c) * C) & a.block_mask)) *
                           rowb;
        r.rows = ok ? r.rows : cin;
        r.bytes = ok ? r.bytes : 0u;
      } else if constexpr (PAGED) {
        const uint8_t* row0 = slot_row(a, cin, p.b, p.kvh, static_cast<int64_t>(p.c) * C, rowb);
        r.rows = row0 ? row0 : cin;
        r.bytes = row0 ? r.bytes : 0u;
      } else {
        r.rows = cin + (g * M + p.c * C) * rowb;
      }
    }
    return r;
  };
  // q rows of a chunk's KV head (rows that are padding or not appended read
  // zeros; live = false reads zeros everywhere)
  auto load_q = [&](uint4 (&qv)[ROWS], const ChunkPos& p, bool live) {
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const int t = Q1 ? 0 : r % Q;
      const int g = Q1 ? r : r / Q;
      const bool valid = live && r < R && t < p.n;
      const int64_t row = valid ? (static_cast<int64_t>(p.b) * a.Hq + p.kvh * a.G + g) * Q + t : 0;
      qv[r] = buf_ld16(make_rsrc(qbase + row * KROW, valid ? KROW : 0u), kc * 16u);
    }
  };

  uint4 qf[ROWS];
  uint4 kbuf[16], vbuf[16];
  float o_acc[ROWS][VEC];
  Acc seg_m[ROWS], seg_l[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    seg_m[r] = neg_inf;
    seg_l[r] = 0;
#pragma unroll
    for (int i = 0; i < VEC; i++) o_acc[r][i] = 0.0f;
  }
  load_q(qf, pos, true);
  {
    const RowSrc sk = src_of(pos, x_begin, true, kin, a.new_key, KROW);
    const RowSrc sv = src_of(pos, x_begin, true, vin, a.new_value, VROW);
#pragma unroll
    for (int u = 0; u < UK; u++) kbuf[u] = load_one(sk, u, k_off);
#pragma unroll
    for (int u = 0; u < UV; u++) vbuf[u] = load_one(sv, u, v_off);
  }
  __builtin_amdgcn_sched_barrier(0);

  for (int64_t x = x_begin; x < x_end; x++) {
    const int64_t grp = grp_of(pos);
    const int j0 = j0_of(pos);         // first slot of the chunk
    const int n_all = n_all_of(pos);   // visited slots
    // out of place: every visited row goes to the output cache at slots
    // j0.. (next to the math below, before each register is reloaded); in
    // place this kernel writes no cache row (the combine kernel stores the
    // appended rows)
    const uint32_t kcopy = static_cast<uint32_t>(n_all) * KROW;
    const uint32_t vcopy = static_cast<uint32_t>(n_all) * VROW;

    // ---- the next chunk: its position and sources ----
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
    const bool more = x + 1 < x_end;
    if constexpr (PAGED && FUSED) {
      if (more && x + 1 - blk_base == kWave) fill_blocks(x + 1);
    }
    const RowSrc nk = src_of(nxt, x + 1, more, kin, a.new_key, KROW);
    const RowSrc nv = src_of(nxt, x + 1, more, vin, a.new_value, VROW);

    // ---- K: scores; each group's registers reload the next chunk's K ----
    Acc sc[NG];  // this lane's finished scores: packed row my_row, one per group
    {
      const int t = Q1 ? 0 : my_row % Q;
      const bool row_ok = my_row < R && t < pos.n;
#pragma unroll
      for (int g = 0; g < NG; g++) {
        if constexpr (OOP) {
#pragma unroll
          for (int gu = 0; gu < GU; gu++)
            store_one(kout + (grp * M + j0) * KROW, kcopy,
                      g * GU + gu, k_off, kbuf[g * GU + gu]);
        }
        Acc part[LK];
#pragma unroll
        for (int gu = 0; gu < GU; gu++)
#pragma unroll
          for (int r = 0; r < ROWS; r++) part[gu * ROWS + r] = Mth::dot(qf[r], kbuf[g * GU + gu]);
#pragma unroll
        for (int gu = 0; gu < GU; gu++) kbuf[g * GU + gu] = load_one(nk, g * GU + gu, k_off);
        __builtin_amdgcn_sched_barrier(0);
        reduce_scatter<LK / 2, LK>(part, kc);
        // visible: an existing row whose token t is appended (t < n) and
        // slot j0 + jl <= len + t
        const int jl = (g * GU + kc / ROWS) * SPLK + ks;
        const bool ok = row_ok && jl < n_all && j0 + jl <= pos.len + t;
        sc[g] = ok ? part[0] * scale : neg_inf;
      }
    }
    // q is dead until the next chunk's scores: reload it for that chunk now
    // (the same rows unless the KV head changes; they stay in the caches)
    load_q(qf, nxt, more);
    __builtin_amdgcn_sched_barrier(0);

    // ---- chunk statistics per row, segment update ----
    Acc m_c[ROWS], l_c[ROWS];
    {
      Acc mloc = sc[0];
#pragma unroll
      for (int g = 1; g < NG; g++) mloc = sc[g] > mloc ? sc[g] : mloc;
      rows_finish<ROWS, true>(rot_reduce<ROWS, true>(mloc), m_c);
    }
    Acc my_m = m_c[0];
#pragma unroll
    for (int r = 1; r < ROWS; r++) my_m = my_row == r ? m_c[r] : my_m;
    Acc p[NG];
    {
      Acc lloc = 0;
#pragma unroll
      for (int g = 0; g < NG; g++) {
        p[g] = sc[g] == neg_inf ? Acc(0) : acc_exp(sc[g] - my_m);
        lloc += p[g];
      }
      rows_finish<ROWS, false>(rot_reduce<ROWS, false>(lloc), l_c);
    }
    Acc alpha[ROWS], beta[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const Acc m_new = m_c[r] > seg_m[r] ? m_c[r] : seg_m[r];
      alpha[r] = seg_m[r] == neg_inf ? Acc(0) : acc_exp(seg_m[r] - m_new);
      beta[r] = m_c[r] == neg_inf ? Acc(0) : acc_exp(m_c[r] - m_new);
      seg_l[r] = seg_l[r] * alpha[r] + l_c[r] * beta[r];
      seg_m[r] = m_new;
      const int t = Q1 ? 0 : r % Q;
      if (r < R && t < pos.n && lane == 0) {
        double* cm = a.ws_chunk_ml + ((grp * a.nchunk_max + pos.c) * R + r) * 2;
        cm[0] = static_cast<double>(m_c[r]);
        cm[1] = static_cast<double>(l_c[r]);
      }
    }
    // attention values exp(s - m_c) and context weights p * beta into the tiles
    {
      Acc my_beta = beta[0];
#pragma unroll
      for (int r = 1; r < ROWS; r++) my_beta = my_row == r ? beta[r] : my_beta;
#pragma unroll
      for (int g = 0; g < NG; g++) {
        const int u = g * GU + kc / ROWS;  // load index of this lane's slot
        const int jl = u * SPLK + ks;
        Elem<T>::store(atile + my_row * C + jl, p[g]);
        if constexpr (kBf16) {
          uint16_t* ph = reinterpret_cast<uint16_t*>(ptile);
          ph[(((u / 2) * SPLV + ks) * ROWS + my_row) * 2 + (u & 1)] =
              f32_to_bf16(static_cast<float>(p[g] * my_beta));
        } else {
          reinterpret_cast<float*>(ptile)[my_row * C + jl] = static_cast<float>(p[g] * my_beta);
        }
      }
    }
    wave_lds_sync();
    // attention rows of the chunk: lane takes AVEC consecutive slots of one
    // packed row (the head's R rows are contiguous: row r = g * Q + t)
    {
      const int64_t head0 = (static_cast<int64_t>(pos.b) * a.Hq + pos.kvh * a.G) * Q;
      T* abase = att + head0 * M + j0;
      const bool vec16 = (reinterpret_cast<uintptr_t>(abase) & 15u) == 0 && (M % AVEC) == 0;
#pragma unroll
      for (int gi = lane; gi < ROWS * C / AVEC; gi += kWave) {
        const int r = gi / (C / AVEC), s0 = (gi % (C / AVEC)) * AVEC;
        const int t = Q1 ? 0 : r % Q;
        if (r < R && t < pos.n && s0 < n_all && !a.read_only) {
          T* dst = abase + static_cast<int64_t>(r) * M + s0;
          if (vec16 && s0 + AVEC <= n_all) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(atile + r * C + s0);
          } else {
            for (int k = 0; k < AVEC && s0 + k < n_all; k++) dst[k] = atile[r * C + s0 + k];
          }
        }
      }
    }

    // ---- V: context partials; each pair's registers reload the next V ----
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const float al = static_cast<float>(alpha[r]);
#pragma unroll
      for (int i = 0; i < VEC; i++) o_acc[r][i] *= al;
    }
    if constexpr (kBf16) {
#pragma unroll
      for (int j = 0; j < UV / 2; j++) {
        if constexpr (OOP) {
          store_one(vout + (grp * M + j0) * VROW, vcopy, 2 * j,
                    v_off, vbuf[2 * j]);
          store_one(vout + (grp * M + j0) * VROW, vcopy, 2 * j + 1,
                    v_off, vbuf[2 * j + 1]);
        }
        uint32_t pp[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; r++) pp[r] = ptile[(j * SPLV + vs) * ROWS + r];
        // (v[slot 2j][d], v[slot 2j+1][d]) for d = 2e (lo) and d = 2e + 1 (hi)
        const uint32_t w0[4] = {vbuf[2 * j].x, vbuf[2 * j].y, vbuf[2 * j].z, vbuf[2 * j].w};
        const uint32_t w1[4] = {vbuf[2 * j + 1].x, vbuf[2 * j + 1].y, vbuf[2 * j + 1].z,
                                vbuf[2 * j + 1].w};
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          lo[e] = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
          hi[e] = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
        }
        // the registers are free again: the next chunk's V goes into them
        // (a load into a register still in use would need a copy per chunk)
        vbuf[2 * j] = load_one(nv, 2 * j, v_off);
        vbuf[2 * j + 1] = load_one(nv, 2 * j + 1, v_off);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 4; e++) {
#pragma unroll
          for (int r = 0; r < ROWS; r++) {
            o_acc[r][2 * e] = Mth::dot2(pp[r], lo[e], o_acc[r][2 * e]);
            o_acc[r][2 * e + 1] = Mth::dot2(pp[r], hi[e], o_acc[r][2 * e + 1]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < UV; u++) {
        if constexpr (OOP)
          store_one(vout + (grp * M + j0) * VROW, vcopy, u, v_off,
                    vbuf[u]);
        const int jl = u * SPLV + vs;
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
          const float pr = reinterpret_cast<const float*>(ptile)[r * C + jl];
          o_acc[r][0] += pr * __uint_as_float(vbuf[u].x);
          o_acc[r][1] += pr * __uint_as_float(vbuf[u].y);
          o_acc[r][2] += pr * __uint_as_float(vbuf[u].z);
          o_acc[r][3] += pr * __uint_as_float(vbuf[u].w);
        }
        vbuf[u] = load_one(nv, u, v_off);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wave_lds_sync();  // the next chunk overwrites the tile

    // ---- flush the segment when the KV head changes or at the end ----
    if (group_ends || !more) {
      // sum o over the lanes that hold the same dims
#pragma unroll
      for (int off = LV; off < kWave; off <<= 1)
#pragma unroll
        for (int r = 0; r < ROWS; r++)
#pragma unroll
          for (int i = 0; i < VEC; i++) o_acc[r][i] += __shfl_xor(o_acc[r][i], off);
      const int64_t seg = w + grp;
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
    pos = nxt;
  }
}

}  // namespace kvc
