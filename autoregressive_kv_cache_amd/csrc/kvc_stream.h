// kvc_stream.h -- stream-mode attend kernel for bf16 decode-shaped steps
// (at most 15 packed query rows per KV head, D = Dv in {64, 128}).
//
// Work split (as attend_decode_kernel, kvc_decode.h): the visible slots of
// every (batch row, KV head) are cut into chunks of 64 slots -- the cached
// slots, then one chunk with the appended rows read from new_key/new_value
// (stream_chunks) -- and the flattened chunk list is cut into contiguous
// ranges, one per stream worker (worker_start: even shares, or, were a unit
// to hold two workgroups, `lead`/8 times the share for the first half of
// the grid).  A worker is one wave holding up to
// ROWS packed rows, or, past 8 rows (GROUPS), two waves side by side that
// read the same chunks and hold 8 rows each.  A worker keeps running
// statistics across the chunks of one KV head (a segment).
//
// What it leaves for the combine kernel (kvc_combine_stream.h), in the
// workspace, indexed by the flattened chunk x or the segment id:
//   ws_pexp[x][r][64]  exp2(s - m_ref) of every slot of the chunk (bf16),
//   ws_cref[x][r]      the reference m_ref those values use (log2 units),
//   ws_seg2[seg][r]    the segment's (m_ref, l) and ws_seg_o[seg][r][Dv] its
//                      unnormalised context sum_j exp2(s_j - m_ref) v_j.
//
// What shapes the kernel is the memory system: the K/V stream is the step's
// bytes, and writes that reach memory while other waves stream cost several
// times their size in read time.  So a wave keeps everything it produces in
// LDS (a stash of its chunks' exp values and references and its segment
// partials) and writes it out once, as one contiguous run, when its range
// is done (or when the stash fills).  The per-chunk work:
//   - K rows are spread over 8 lanes per slot (each 16-byte load still
//     covers eight whole 128-byte lines): lane l holds dims
//     [h*64 + (l>>3)*8, +8) of slot 8k + (l&7) for load k*NH + h.  The 8
//     partial dot products of a slot are finished by a reduce-scatter over
//     lane bits 5, 4 (v_permlane32_swap / v_permlane16_swap: one exchange
//     and one add per pair of partials) and 3 (DPP), after which lane l
//     holds the scores of slot l for every packed row;
//   - the running maximum is a lazy reference: it is raised (with the
//     rescaling of the running sum and context) only when some score
//     exceeds it by more than 2^8 in the exponent, so most chunks take no
//     cross-lane reduction at all; exp2(s - m_ref) <= 2^8 holds fine in
//     fp32 and bf16, and the combine rescales each chunk by its own
//     reference, so the result is the same softmax;
//   - the context weights go through a small LDS tile to the V layout (lane
//     l holds 8 dims of slot SPLV*u + l/LV for load u).
//
// The step follows "Autoregressive KV-cache append and causal attention",
// Required behavior: KV head floor(h / (Hq/Hk)), slot length + t for
// appended row t, visibility j <= length + t (lower-right alignment,
// KempnerForge PR 542, Summary), scores scale * dot(q, k) and a
// max-subtracted softmax.  Paged caches ("ClikaRT::ops::attention_over_cache",
// function description) change only where a chunk's rows are read.
#pragma once

#include "kvc_decode.h"

namespace kvc {

// A score more than 2^kLazyMargin above the reference raises it.
constexpr float kLazyMargin = 8.0f;
constexpr float kLog2e = 1.4426950408889634f;
// Reference before a segment's first visible score: finite, so that
// exp2(-inf - reference) is 0 and not NaN.
constexpr float kRefFloor = -1.0e30f;
constexpr int kStreamChunk = 64;

// One worker wave per SIMD (one workgroup of 4 waves per compute unit), for
// 4 rows as for 8.  Measured at B = 32, Hq = 32, Hk = 8, 8192 slots (4
// rows): two 4-row waves per SIMD (two workgroups per unit, the first one
// placed taking twice the share) 109.7 us per step against 107.4 with one;
// at twice the batch 207.3 against 200.5.  With one wave per SIMD no wave
// has an older neighbour that wins the issue arbitration, and a chunk of K
// and V in flight per wave (128 KB per unit) keeps the stream going.
template <int ROWS>
constexpr int stream_waves_per_simd() {
  return 1;
}
// Chunks a wave keeps in LDS before it writes them out (the LDS of a unit
// holds one workgroup's stashes: 4 x 48 chunks of 4 rows, or 4 x 24 of 8).
// A wave whose range fits its stash writes it once, when the range ends;
// with 4 rows 48 chunks were 4 us per step faster than 24 at twice the
// decode batch (37 chunks a worker) and level at the decode batch.
template <int ROWS>
constexpr int stream_stash_chunks() {
  return ROWS > 4 ? 24 : 48;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Sums across 32-lane halves (lane bit 5) or 16-lane rows (bit 4): the
// upper half of `lo` is swapped with the lower half of `hi` (permlane32), or
// the odd rows of `lo` with the even rows of `hi` (permlane16), and the two
// are added.  Lanes with the bit clear get lo + partner's lo, the others
// hi + partner's hi; with lo == hi every lane gets the pair's sum.
__device__ __forceinline__ float sum_swap32(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_swap16(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reduce (max or sum) over all 64 lanes; every lane gets the result.
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  v = op(v, dpp<dpp_row_ror(8)>(v));
  v = op(v, dpp<dpp_row_ror(4)>(v));
  v = op(v, dpp<dpp_row_ror(2)>(v));
  v = op(v, dpp<dpp_row_ror(1)>(v));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Workspace stores through a scalar descriptor: the address is the
// descriptor's base plus a 32-bit lane offset, so no 64-bit per-lane address
// has to stay live across the kernel's loop.  POLICY is the store's cache
// operand: 0 (the default: the line stays in the XCD's L2 until it is
// evicted or the kernel ends) or kDeviceScope (the sc1 bit: device-scope
// coherence, so the store is written through the L2 as it happens).
constexpr int kDeviceScope = 16;
template <int V>
struct StorePolicy {
  static constexpr int value = V;
};
template <int POLICY>
__device__ __forceinline__ void ws_st16(__amdgpu_buffer_rsrc_t r, uint32_t off, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, static_cast<int>(off), 0, POLICY);
}
template <int POLICY>
__device__ __forceinline__ void ws_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, static_cast<int>(off), 0, POLICY);
}
// The workspace stores are written through (kDeviceScope) when a KV head
// packs 8 rows or more, or when the launch's exp values pass this many
// bytes; otherwise they keep the default policy.  Measured per step: with 4
// rows per KV head and 8.2 MiB of exp values (B = 32, 8192 slots) the
// default is 2.5 us faster, and so it is for the paged step and
// re-attention there; from 16.3 MiB on (twice the batch; twice the
// capacity: 18 MiB; 131072 slots: 24 MiB) writing through is 2-4 % faster;
// with 8 rows (16384 or 131072 slots) and 12 rows it is up to 4 % faster,
// and never slower.  The bound sits between the measured sizes.
constexpr int64_t kStashWriteThroughBytes = int64_t{12} << 20;

template <int D, int DV, int ROWS, bool Q1, bool OOP, bool FUSED, bool PAGED, bool GROUPS>
__global__ __launch_bounds__(kDecodeThreads)
__attribute__((amdgpu_waves_per_eu(stream_waves_per_simd<ROWS>()))) void attend_stream_kernel(
    StepArgs a, const int64_t* __restrict__ rowinfo, const int32_t* __restrict__ wstart) {
  using Mth = DecodeMath<bf16>;
  constexpr int C = kStreamChunk;              // slots per chunk
  constexpr int KROW = D * 2, VROW = DV * 2;   // row bytes
  constexpr int NH = KROW / 128;               // 128-byte segments per K row
  constexpr int UK = 8 * NH;                   // K loads per lane per chunk
  constexpr int LV = VROW / 16, SPLV = kWave / LV;  // lanes per V row, V rows per load
  constexpr int UV = C / SPLV;                 // V loads per lane per chunk
  constexpr int NPV = UV / 2;                  // slot pairs per lane in the context products
  constexpr int S = stream_stash_chunks<ROWS>();
  static_assert(KROW % 128 == 0 && NH >= 1 && NH <= 2, "K rows of 128 or 256 bytes");
  static_assert(SPLV * VROW == 1024 && UV % 2 == 0 && UV <= 16, "V rows of 128 or 256 bytes");
  static_assert(ROWS == 4 || ROWS == 8, "packed rows per wave");
  static_assert(!(PAGED && OOP), "the paged cache is updated in place");

  // per wave: context weights, bf16 pairs [slot lane s][pair m][row] ->
  // (slot 2*SPLV*m + s, slot 2*SPLV*m + SPLV + s); the stash of exp values
  // [chunk][row][slot] and references [chunk][row]; stashed segment partials
  __shared__ uint32_t pw_all[kDecodeWaves][SPLV * ROWS * NPV];
  __shared__ __align__(16) uint16_t xs_all[kDecodeWaves][S][ROWS * C];
  __shared__ float xr_all[kDecodeWaves][S][ROWS];
  constexpr int RT = FUSED ? kDecodeFusedRows : 1;
  __shared__ int32_t rt_len[RT], rt_n[RT];
  __shared__ int64_t rt_first[RT];
  __shared__ int64_t rt_total;
  __shared__ int32_t blk_all[(PAGED && FUSED) ? kDecodeWaves : 1][kWave];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  uint32_t* pw = pw_all[wave];
  uint16_t(*xs)[ROWS * C] = xs_all[wave];
  float(*xr)[ROWS] = xr_all[wave];
  const uint32_t k_off = static_cast<uint32_t>((lane & 7) * KROW + (lane >> 3) * 16);
  const uint32_t v_off = static_cast<uint32_t>(lane * 16);
  const float scale_l2 = static_cast<float>(a.scale) * kLog2e;
  const int Q = Q1 ? 1 : static_cast<int>(a.Q);
  const int R = static_cast<int>(a.R);
  const int Hk = static_cast<int>(a.Hk);
  const int64_t M = a.M;
  // Row groups (more packed rows than a wave holds): a KV head's R packed
  // rows are cut into groups of ROWS, one wave each; the waves of one
  // stream worker (rg_waves of them, side by side in the workgroup, a power
  // of two) walk the same chunk range.  Their K/V loads use the default
  // cache policy, so that the unit's caches serve a chunk's rows to the
  // later waves (non-temporal loads would send each group to memory: 1.8x
  // the time at 8 rows in two groups of 4).  Waves past the last group have
  // no rows.
  // (GROUPS false: one group, rows [0, R), R <= ROWS)
  const int RGW = GROUPS ? a.rg_waves : 1;
  const int r0 = GROUPS ? (wave % RGW) * ROWS : 0;  // the group's first packed row
  const int NR = GROUPS ? (R - r0 < ROWS ? R - r0 : ROWS) : R;  // rows of the group (<= 0: none)

  // ---- row information (as attend_decode_kernel) ----
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
  const int64_t w = blockIdx.x * static_cast<int64_t>(kDecodeWaves / RGW) + wave / RGW;
  if (w >= Pw || (GROUPS && NR <= 0)) return;
  const bool write_through = R >= 8 || Nc * R * C * 2 > kStashWriteThroughBytes;
  const int32_t lead = effective_lead(Nc, Pw, a.lead);
  const int64_t x_begin = worker_start(w, Nc, Pw, lead), x_end = worker_start(w + 1, Nc, Pw, lead);
  if (x_begin >= x_end) return;

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

  auto grp_of = [&](const ChunkPos& p) { return static_cast<int64_t>(p.b) * Hk + p.kvh; };
  auto is_new_of = [&](const ChunkPos& p) { return p.c == p.nc - 1; };
  auto j0_of = [&](const ChunkPos& p) { return is_new_of(p) ? p.len : p.c * C; };
  auto n_all_of = [&](const ChunkPos& p) {
    return is_new_of(p) ? p.n : (p.c * C + C < p.len ? C : p.len - p.c * C);
  };
  // Paged and FUSED: the wave keeps the blocks of its next 64 chunks in LDS
  // (entry i: chunk blk_base + i, filled once per 64 chunks); otherwise each
  // chunk reads its table entry.  A chunk lies inside one block (blocks hold
  // a power of two >= 64 slots), so its rows are contiguous; an entry outside
  // the pool reads as zero rows.
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
  // V load u of a chunk (as load_one, kvc_decode.h; cache policy as for K)
  auto load_v = [&](const RowSrc& s, int u, uint32_t lane_off) {
    const uint32_t base = static_cast<uint32_t>(u / 4) * 4096u;
    const uint32_t imm = static_cast<uint32_t>(u % 4) * 1024u;
    const uint32_t left = s.bytes > base ? s.bytes - base : 0u;
    return buf_ld16<GROUPS ? 0 : kNonTemporal>(make_rsrc(s.rows + base, left), lane_off + imm);
  };
  // K load (k, h): slot 8k + (lane & 7), bytes [h*128 + (lane>>3)*16, +16);
  // the descriptor starts at the 8-slot group so the lane offset stays small
  auto load_k = [&](const RowSrc& s, int k, int h) {
    const uint32_t base = static_cast<uint32_t>(k) * 8u * KROW;
    const uint32_t left = s.bytes > base ? s.bytes - base : 0u;
    return buf_ld16<GROUPS ? 0 : kNonTemporal>(make_rsrc(s.rows + base, left), k_off + h * 128u);
  };
  auto store_k = [&](uint8_t* out, uint32_t bytes, int k, int h, const uint4& v) {
    const uint32_t base = static_cast<uint32_t>(k) * 8u * KROW;
    const uint32_t left = bytes > base ? bytes - base : 0u;
    buf_st16(make_rsrc(out + base, left), k_off + h * 128u, v);
  };
  // q slices of a chunk's KV head: qv[r][h] = dims [h*64 + (lane>>3)*8, +8)
  // of packed row r (zeros for padding rows and rows that append nothing)
  auto load_q = [&](uint4 (&qv)[ROWS][NH], const ChunkPos& p) {
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const int t = Q1 ? 0 : (r0 + r) % Q;
      const int g = Q1 ? r0 + r : (r0 + r) / Q;
      const bool valid = r < NR && t < p.n;
      const int64_t row = valid ? (static_cast<int64_t>(p.b) * a.Hq + p.kvh * a.G + g) * Q + t : 0;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(qbase + row * KROW, valid ? KROW : 0u);
#pragma unroll
      for (int h = 0; h < NH; h++)
        qv[r][h] = buf_ld16(rs, static_cast<uint32_t>(h * 128 + (lane >> 3) * 16));
    }
  };

  // ---- the stash: exp values and references of chunks [xs0, xs0 + ns) ----
  int64_t xs0 = x_begin;
  int ns = 0;
  auto flush_stash = [&]() {
    if (a.read_only) {  // re-attention: the exp values serve only the attention rows
      xs0 += ns;
      ns = 0;
      return;
    }
    wave_lds_sync();
    auto put = [&](auto pol) {
      constexpr int POL = decltype(pol)::value;
      // exp values: ns chunks of R rows of C bf16 in the workspace; with row
      // groups, this group's NR rows of each (one contiguous run per chunk)
      if constexpr (GROUPS) {
        const int pieces = ns * NR * (C / 8);
        const __amdgpu_buffer_rsrc_t dx =
            make_rsrc(a.ws_pexp + xs0 * R * C, static_cast<uint32_t>(ns * R * C) * 2u);
        for (int p = lane; p < pieces; p += kWave) {
          const int i = p / (NR * (C / 8)), rr = (p / (C / 8)) % NR, s8 = p % (C / 8);
          ws_st16<POL>(dx, static_cast<uint32_t>(((i * R + r0 + rr) * (C / 8) + s8) * 16),
                  *reinterpret_cast<const uint4*>(&xs[i][rr * C + s8 * 8]));
        }
        const __amdgpu_buffer_rsrc_t dr =
            make_rsrc(a.ws_cref + xs0 * R, static_cast<uint32_t>(ns * R) * 4u);
        for (int p = lane; p < ns * NR; p += kWave)
          ws_st4<POL>(dr, static_cast<uint32_t>((p / NR) * R + r0 + p % NR) * 4u, xr[p / NR][p % NR]);
      } else {
        const int pieces = ns * R * (C / 8);
        const __amdgpu_buffer_rsrc_t dx =
            make_rsrc(a.ws_pexp + xs0 * R * C, static_cast<uint32_t>(pieces) * 16u);
        for (int p = lane; p < pieces; p += kWave) {
          const int i = p / (R * (C / 8)), rr = (p / (C / 8)) % R, s8 = p % (C / 8);
          ws_st16<POL>(dx, static_cast<uint32_t>(p) * 16u,
                  *reinterpret_cast<const uint4*>(&xs[i][rr * C + s8 * 8]));
        }
        const __amdgpu_buffer_rsrc_t dr =
            make_rsrc(a.ws_cref + xs0 * R, static_cast<uint32_t>(ns * R) * 4u);
        for (int p = lane; p < ns * R; p += kWave)
          ws_st4<POL>(dr, static_cast<uint32_t>(p) * 4u, xr[p / R][p % R]);
      }
    };
    if (write_through) put(StorePolicy<kDeviceScope>{}); else put(StorePolicy<0>{});
    xs0 += ns;
    ns = 0;
  };

  uint4 qv[ROWS][NH];
  uint4 kb[UK], vb[UV];
  float o_acc[ROWS][8];
  float mref[ROWS], l_lane[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    mref[r] = kRefFloor;
    l_lane[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) o_acc[r][i] = 0.0f;
  }
  load_q(qv, pos);
  {
    const RowSrc sk = src_of(pos, x_begin, true, kin, a.new_key, KROW);
    const RowSrc sv = src_of(pos, x_begin, true, vin, a.new_value, VROW);
#pragma unroll
    for (int k = 0; k < 8; k++)
#pragma unroll
      for (int h = 0; h < NH; h++) kb[k * NH + h] = load_k(sk, k, h);
#pragma unroll
    for (int u = 0; u < UV; u++) vb[u] = load_v(sv, u, v_off);
  }
  __builtin_amdgcn_sched_barrier(0);

  // this lane's place in the context-weight tile, and its slot lane in the V layout
  const int ps = lane % SPLV, ph = (lane / SPLV) & 1, pm = lane / (2 * SPLV);
  const int rs = lane / LV;

  for (int64_t x = x_begin; x < x_end; x++) {
    if (ns == S) flush_stash();
    const int64_t grp = grp_of(pos);
    const int j0 = j0_of(pos);
    const int n_all = n_all_of(pos);
    const uint32_t kcopy = static_cast<uint32_t>(n_all) * KROW;
    const uint32_t vcopy = static_cast<uint32_t>(n_all) * VROW;

    // ---- the next chunk ----
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

    // ---- scores ----
    // Partial dot products of 8-slot group k, reduced as soon as their
    // partners exist: v_permlane32_swap pairs k with k + 4 (lane bit 5),
    // v_permlane16_swap pairs the results for k and k + 2 (bit 4), DPP the
    // last two (bit 3).  Lane l ends with the scores of slot l.  Each group's
    // K registers reload the next chunk's rows once they are consumed.
    auto partials = [&](int k, float (&out)[ROWS]) {
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        float acc = Mth::dot(qv[r][0], kb[k * NH]);
        if constexpr (NH == 2) {
          acc = Mth::dot2(qv[r][1].x, kb[k * NH + 1].x, acc);
          acc = Mth::dot2(qv[r][1].y, kb[k * NH + 1].y, acc);
          acc = Mth::dot2(qv[r][1].z, kb[k * NH + 1].z, acc);
          acc = Mth::dot2(qv[r][1].w, kb[k * NH + 1].w, acc);
        }
        out[r] = acc;
      }
      if constexpr (OOP) {
#pragma unroll
        for (int h = 0; h < NH; h++)
          store_k(kout + (grp * M + j0) * KROW, kcopy, k, h, kb[k * NH + h]);
      }
#pragma unroll
      for (int h = 0; h < NH; h++) kb[k * NH + h] = load_k(nk, k, h);
    };
    float s5[4][ROWS], s4[2][ROWS], sc[ROWS];
    constexpr int kOrder[4] = {0, 2, 1, 3};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int kl = kOrder[i];
      float pa[ROWS], pb[ROWS];
      partials(kl, pa);
      partials(kl + 4, pb);
#pragma unroll
      for (int r = 0; r < ROWS; r++) s5[kl][r] = sum_swap32(pa[r], pb[r]);
      if (i == 1 || i == 3) {
        const int k2 = i == 1 ? 0 : 1;
#pragma unroll
        for (int r = 0; r < ROWS; r++) s4[k2][r] = sum_swap16(s5[k2][r], s5[k2 + 2][r]);
      }
    }
    {
      const bool upper = (lane & 8) != 0;
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        const float send = upper ? s4[0][r] : s4[1][r], keep = upper ? s4[1][r] : s4[0][r];
        sc[r] = keep + dpp<dpp_row_ror(8)>(send);
      }
    }
    // q of the next chunk (a new KV head only)
    if (group_ends && more) load_q(qv, nxt);
    __builtin_amdgcn_sched_barrier(0);

    // ---- visibility, lazy reference, exponentials ----
    const int jl = lane;  // this lane's slot in the chunk
    bool big = false;
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      const int t = Q1 ? 0 : (r0 + r) % Q;
      const bool vis = r < NR && t < pos.n && jl < n_all && j0 + jl <= pos.len + t;
      sc[r] = vis ? sc[r] * scale_l2 : -INFINITY;
      big = big || sc[r] > mref[r] + kLazyMargin;
    }
    if (__builtin_amdgcn_ballot_w64(big) != 0) {
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        const float m_new = fmaxf(mref[r], wave_reduce<true>(sc[r]));
        const float alpha = exp2_fast(mref[r] - m_new);
        l_lane[r] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; i++) o_acc[r][i] *= alpha;
        mref[r] = m_new;
      }
    }
    {
      uint16_t* pwh = reinterpret_cast<uint16_t*>(pw);
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        const float p = exp2_fast(sc[r] - mref[r]);
        l_lane[r] += p;
        const uint16_t pb = bf16_bits(p);
        xs[ns][r * C + jl] = pb;
        pwh[((ps * NPV + pm) * ROWS + r) * 2 + ph] = pb;
      }
      // every lane writes the reference of row lane % ROWS (no branch)
      float mine = mref[0];
#pragma unroll
      for (int r = 1; r < ROWS; r++) mine = (lane & (ROWS - 1)) == r ? mref[r] : mine;
      xr[ns][lane & (ROWS - 1)] = mine;
    }
    wave_lds_sync();

    // ---- context: o += p * v over slot pairs; each pair's registers reload the next V ----
#pragma unroll
    for (int m = 0; m < NPV; m++) {
      uint32_t pr[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; r++) pr[r] = pw[(rs * NPV + m) * ROWS + r];
      if constexpr (OOP) {
        store_one(vout + (grp * M + j0) * VROW, vcopy, 2 * m, v_off, vb[2 * m]);
        store_one(vout + (grp * M + j0) * VROW, vcopy, 2 * m + 1, v_off, vb[2 * m + 1]);
      }
      const uint32_t w0[4] = {vb[2 * m].x, vb[2 * m].y, vb[2 * m].z, vb[2 * m].w};
      const uint32_t w1[4] = {vb[2 * m + 1].x, vb[2 * m + 1].y, vb[2 * m + 1].z,
                              vb[2 * m + 1].w};
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        lo[e] = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
        hi[e] = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
      }
      vb[2 * m] = load_v(nv, 2 * m, v_off);
      vb[2 * m + 1] = load_v(nv, 2 * m + 1, v_off);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int e = 0; e < 4; e++) {
#pragma unroll
        for (int r = 0; r < ROWS; r++) {
          o_acc[r][2 * e] = Mth::dot2(pr[r], lo[e], o_acc[r][2 * e]);
          o_acc[r][2 * e + 1] = Mth::dot2(pr[r], hi[e], o_acc[r][2 * e + 1]);
        }
      }
    }
    wave_lds_sync();  // the next chunk overwrites the tile
    ns++;

    // ---- close the segment when the KV head changes or at the end ----
    if (group_ends || !more) {
      // sum o over the lanes that hold the same dims (lane bits 5, 4 and,
      // for 128-byte V rows, 3)
      // (one row at a time: the loads in flight keep most registers busy)
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
          float v = o_acc[r][i];
          if constexpr (LV == 8) v += dpp<dpp_row_ror(8)>(v);
          v = sum_swap16(v, v);
          o_acc[r][i] = sum_swap32(v, v);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      float l_seg[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        l_seg[r] = wave_reduce<false>(l_lane[r]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int64_t seg = w + grp;
      // this group's rows r0 .. r0 + NR - 1; rows >= NR fall outside the
      // descriptors and are not stored
      const __amdgpu_buffer_rsrc_t so_rs =
          make_rsrc(a.ws_seg_o + (seg * R + r0) * DV, static_cast<uint32_t>(NR * DV) * 4u);
      const __amdgpu_buffer_rsrc_t sm_rs =
          make_rsrc(a.ws_seg2 + (seg * R + r0) * 2, static_cast<uint32_t>(NR * 2) * 4u);
      float mv = mref[0], lv = l_seg[0];
#pragma unroll
      for (int r = 1; r < ROWS; r++) {
        mv = (lane >> 1) == r ? mref[r] : mv;
        lv = (lane >> 1) == r ? l_seg[r] : lv;
      }
      auto put = [&](auto pol) {
        constexpr int POL = decltype(pol)::value;
        if (rs == 0) {
#pragma unroll
          for (int r = 0; r < ROWS; r++) {
            const uint32_t off = static_cast<uint32_t>(r * DV + lane * 8) * 4u;
            ws_st16<POL>(so_rs, off,
                         make_uint4(__float_as_uint(o_acc[r][0]), __float_as_uint(o_acc[r][1]),
                                    __float_as_uint(o_acc[r][2]), __float_as_uint(o_acc[r][3])));
            ws_st16<POL>(so_rs, off + 16u,
                         make_uint4(__float_as_uint(o_acc[r][4]), __float_as_uint(o_acc[r][5]),
                                    __float_as_uint(o_acc[r][6]), __float_as_uint(o_acc[r][7])));
          }
        }
        if (lane < 2 * ROWS) ws_st4<POL>(sm_rs, static_cast<uint32_t>(lane) * 4u, lane & 1 ? lv : mv);
      };
      if (write_through) put(StorePolicy<kDeviceScope>{}); else put(StorePolicy<0>{});
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        mref[r] = kRefFloor;
        l_lane[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) o_acc[r][i] = 0.0f;
      }
    }
    pos = nxt;
  }
  flush_stash();
}

}  // namespace kvc
