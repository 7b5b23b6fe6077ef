// kvc_common.h -- device-side types and helpers shared by the step's
// kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int kWave = 64;

// bfloat16 storage word (the top 16 bits of a binary32).
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// binary32 -> bfloat16 with round-to-nearest-even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Element traits: storage type T, accumulation type Acc.  fp32 inputs
// accumulate in fp64 (scores reach ~1e3 and the probabilities must hold to
// 1e-5); bf16 inputs accumulate in fp32.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  using Acc = double;
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static double load(const float* p) { return static_cast<double>(*p); }
  __device__ __forceinline__ static void store(float* p, double v) { *p = static_cast<float>(v); }
  __device__ __forceinline__ static float zero() { return 0.0f; }
};

template <>
struct Elem<bf16> {
  using Acc = float;
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const bf16* p) { return bf16_to_f32(p->bits); }
  __device__ __forceinline__ static void store(bf16* p, float v) { p->bits = f32_to_bf16(v); }
  __device__ __forceinline__ static bf16 zero() { return bf16{0}; }
};

__device__ __forceinline__ double acc_exp(double x) { return exp(x); }
__device__ __forceinline__ float acc_exp(float x) { return __expf(x); }

// Everything one step's kernels need; passed by value as the kernel argument.
//
// Work is cut into chunks of C cache slots per (batch row b, KV head h).
// Dense mode: chunk c of group g = b * Hk + h covers slots
// [c*C, min((c+1)*C, len+n)).  Stream mode: see stream_chunks (the cached
// slots in chunks of C, then one chunk of the appended rows).
// For every chunk the attend kernel leaves, per packed query row r,
//   chunk statistics  m_c = max_j s_j,  l_c = sum_j exp(s_j - m_c),
//   exp(s_j - m_c) in the attention buffer,
// and per segment (a run of chunks of one group processed by one workgroup)
//   m_seg, l_seg and o_seg = sum_j exp(s_j - m_seg) v_j.
// Segments are addressed in one of two ways:
//   seg_mode 0 ("dense"): one segment per chunk, id = g * nchunk_max + c;
//   seg_mode 1 ("stream"): worker w of Pe = min(P, Nc) (a wave) owns the
//     chunk range [floor(w*Nc/Pe), floor((w+1)*Nc/Pe)) of the flattened
//     chunk list -- never empty, as Pe <= Nc -- and its segment of group g
//     has id w + g (unique: along the chunk list g and w never decrease and
//     one of them grows between distinct pairs).  The segments of a group
//     are therefore the consecutive ids of the workers owning its chunks.
struct StepArgs {
  int64_t B, Hq, Hk, Q, M, D, Dv;
  int32_t G;          // Hq / Hk
  int32_t R;          // packed rows per KV head = G * Q (row r = g * Q + t)
  int32_t rows_per_tile;
  int32_t row_tiles;
  int64_t C;          // slots per chunk (a power of two)
  int32_t C_log2;     // log2(C)
  int64_t nchunk_max; // ceil(M / C)
  int64_t CS;         // slots per combine workgroup (a multiple of C)
  int64_t P;          // stream workers (waves of the attend grid, stream mode)
  int32_t lead;       // stream shares: weight, in eighths, of the workers in the first half of the grid
  int32_t seg_mode;   // 0 dense, 1 stream, 2 stream with the bf16 stream kernel's workspace
  int32_t combine_copies_tail;  // out of place: combine copies slots the attend kernel skips
  double scale;       // resolved softmax scale
  int64_t elem_bytes; // 4 (fp32) or 2 (bf16)
  int32_t out_of_place;
  const void* query;
  const void* new_key;
  const void* new_value;
  const void* kc_in;  // cache read for slots < length (== kc_out in place)
  const void* vc_in;
  void* kc_out;       // cache written (copy + new rows, or new rows only)
  void* vc_out;
  const int64_t* lengths;
  const uint8_t* mask;
  void* attention;
  void* context;
  int64_t* lengths_out;
  int32_t* row_status;
  int64_t* ws_hdr;       // [8]: [0] total chunk count Nc, [1] busy workers Pe (stream mode)
  int64_t* ws_rowinfo;   // [B][4]: length, n, status, first chunk index (stream mode)
  double* ws_chunk_ml;   // [B*Hk][nchunk_max][R][2]: m_c, l_c
  double* ws_seg_ml;     // [nseg][R][2]: m_seg, l_seg
  float* ws_seg_o;       // [nseg][R][Dv]: o_seg
  int32_t* ws_wstart;    // [P][4]: first (b, head, chunk) of each stream worker
  // bf16 stream kernel (kvc_stream.h), indexed by the flattened chunk x:
  uint16_t* ws_pexp;     // [Nc][R][C]: exp2(s - m_ref) of the chunk's slots (bf16)
  float* ws_cref;        // [Nc][R]: the reference m_ref (log2 units) of each chunk
  float* ws_seg2;        // [nseg][R][2]: m (log2 units) and l of each segment
  // paged cache (stream path): kc_in/kc_out and vc_in/vc_out are the block
  // pools [num_blocks][Hk][block_rows][D or Dv]; slot j of batch row b is
  // row j & block_mask of block block_table[b * max_blocks + (j >> block_log2)]
  // (a power-of-two block, or one block of M rows per batch row: log2 62,
  // mask all ones); no table = block b
  int32_t paged;
  int32_t block_log2;
  int64_t block_rows;
  int64_t block_mask;
  int64_t num_blocks;
  int64_t max_blocks;
  const int32_t* block_table;
  // read-only re-attention: no cache slot is written, and the combine adds
  // sinks[query head] (if given) as one more logit to each softmax
  int32_t read_only;
  const float* sinks;
  int32_t rg_waves;   // stream decode: waves per worker (row groups rounded up to 1, 2 or 4)
};

// Block holding slot j of batch row b (paged cache).
__device__ inline int64_t block_of(const StepArgs& a, int64_t b, int64_t j) {
  return a.block_table ? a.block_table[b * a.max_blocks + (j >> a.block_log2)] : b;
}

// Base of cache slot j of (batch row b, KV head h), rows of row_bytes bytes:
// the dense [B][Hk][M] layout, or the paged block pool (nullptr when the
// table entry is outside [0, num_blocks): such rows are neither read nor
// written).
__device__ inline const uint8_t* slot_row(const StepArgs& a, const void* cache, int64_t b,
                                          int64_t h, int64_t j, int64_t row_bytes) {
  const uint8_t* base = static_cast<const uint8_t*>(cache);
  if (!a.paged) return base + ((b * a.Hk + h) * a.M + j) * row_bytes;
  const int64_t blk = block_of(a, b, j);
  if (blk < 0 || blk >= a.num_blocks) return nullptr;
  return base + ((blk * a.Hk + h) * a.block_rows + (j & a.block_mask)) * row_bytes;
}

struct RowInfo {
  int64_t len;     // lengths[b] as given
  int64_t n;       // appended rows (0 on a rejected row)
  int32_t status;  // KVC_ROW_* code
};

// Row preparation for batch row b, run by one full wave (uniform result):
// n = leading run of Trues in append_mask[b,:]; a length outside [0, M], a
// True after a False, or length + n > M rejects the row (n = 0).  The order
// of the checks fixes which code a row with several faults reports.
__device__ inline RowInfo wave_row_info(const int64_t* lengths, const uint8_t* mask, int64_t Q,
                                        int64_t M, int64_t b) {
  const int lane = threadIdx.x & (kWave - 1);
  RowInfo ri;
  ri.len = lengths[b];
  int64_t n = 0;
  bool seen_false = false, not_prefix = false;
  for (int64_t t0 = 0; t0 < Q; t0 += kWave) {
    const int64_t t = t0 + lane;
    const bool v = (t < Q) && (mask[b * Q + t] != 0);
    const uint64_t ones = __ballot(v);
    const int64_t left = Q - t0;
    const uint64_t in_range = left >= kWave ? ~0ull : ((1ull << left) - 1ull);
    const uint64_t falses = ~ones & in_range;
    if (!seen_false) {
      if (falses == 0) {
        n += __popcll(in_range);
      } else {
        const int first_false = __ffsll(static_cast<unsigned long long>(falses)) - 1;
        n += first_false;
        seen_false = true;
        const uint64_t above = first_false >= 63 ? 0ull : (ones >> (first_false + 1));
        if (above != 0) not_prefix = true;
      }
    } else if (ones != 0) {
      not_prefix = true;
    }
  }
  if (ri.len < 0 || ri.len > M) {
    ri.status = 1;
    ri.n = 0;
  } else if (not_prefix) {
    ri.status = 3;
    ri.n = 0;
  } else if (ri.len + n > M) {
    ri.status = 2;
    ri.n = 0;
  } else {
    ri.status = 0;
    ri.n = n;
  }
  return ri;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o);
    v = v > w ? v : w;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of chunks of one batch row's KV head that hold a slot a valid
// query can see (all slots < length + n); 0 when the row appends nothing.
__device__ __forceinline__ int64_t row_chunks(int64_t len, int64_t n, int64_t C) {
  return n > 0 ? ceil_div(len + n, C) : 0;
}

// Stream path: the chunks of one batch row's KV head are the cached slots
// [0, length) cut into ceil(length / C) chunks (the last one partial) and
// one more chunk with the n appended rows (slots [length, length + n), read
// from new_key / new_value); 0 chunks when the row appends nothing.  Slot
// j < length lies in chunk j / C, an appended slot in chunk
// ceil(length / C).
__device__ __forceinline__ int64_t stream_chunks(int64_t len, int64_t n, int64_t C) {
  return n > 0 ? ceil_div(len, C) + 1 : 0;
}
__device__ __forceinline__ int64_t stream_chunk_of(int64_t j, int64_t len, int64_t C) {
  return j < len ? j / C : ceil_div(len, C);
}

// Stream-K shares.  Worker w (workgroup * waves + wave) owns the flattened
// chunks [worker_start(w), worker_start(w + 1)) of the Nc chunks, for
// w < Pe.  With lead == 8 the shares are even: floor(w * Nc / Pe).  With
// another lead, the workers of the first half of the grid (the first
// workgroup placed on each compute unit when the grid holds two per unit)
// take lead / 8 times the share of the others: on a unit the earlier
// workgroup wins most of the memory arbitration, so even shares leave the
// later one finishing alone.  The weights apply only when every worker
// still gets at least one chunk (Nc >= 2 Pe); else the shares are even.
__device__ __forceinline__ int32_t effective_lead(int64_t Nc, int64_t Pe, int32_t lead) {
  return (lead > 8 && Pe >= 2 && Nc >= 2 * Pe) ? lead : 8;
}
// S(w) = lead * min(w, H) + 8 * max(w - H, 0), H = Pe / 2; start = floor(S(w) Nc / S(Pe))
__device__ __forceinline__ int64_t worker_start(int64_t w, int64_t Nc, int64_t Pe, int32_t lead) {
  if (lead == 8) return w * Nc / Pe;
  const int64_t H = Pe / 2;
  const int64_t S = lead * (w < H ? w : H) + 8 * (w > H ? w - H : 0);
  const int64_t T = lead * H + 8 * (Pe - H);
  return S * Nc / T;
}
// The worker whose range holds chunk x (0 <= x < Nc): the largest w < Pe
// with worker_start(w) <= x, i.e. with S(w) <= floor(((x + 1) T - 1) / Nc).
__device__ __forceinline__ int64_t worker_owner(int64_t x, int64_t Nc, int64_t Pe, int32_t lead) {
  if (lead == 8) return ((x + 1) * Pe - 1) / Nc;
  const int64_t H = Pe / 2;
  const int64_t T = lead * H + 8 * (Pe - H);
  const int64_t K = ((x + 1) * T - 1) / Nc;
  const int64_t w = K >= lead * H ? H + (K - lead * H) / 8 : K / lead;
  return w < Pe - 1 ? w : Pe - 1;
}

// Row preparation by one thread (same checks, same order as wave_row_info).
__device__ inline RowInfo thread_row_info(const int64_t* lengths, const uint8_t* mask, int64_t Q,
                                          int64_t M, int64_t b) {
  RowInfo ri;
  ri.len = lengths[b];
  int64_t n = 0;
  while (n < Q && mask[b * Q + n] != 0) n++;
  bool not_prefix = false;
  for (int64_t t = n; t < Q; t++)
    if (mask[b * Q + t] != 0) not_prefix = true;
  if (ri.len < 0 || ri.len > M) {
    ri.status = 1;
    ri.n = 0;
  } else if (not_prefix) {
    ri.status = 3;
    ri.n = 0;
  } else if (ri.len + n > M) {
    ri.status = 2;
    ri.n = 0;
  } else {
    ri.status = 0;
    ri.n = n;
  }
  return ri;
}

}  // namespace kvc
