// kvc_backward.h -- backward of the step for fp32 or bf16 tensors (the math
// runs in fp32 and fp64 either way; each gradient is rounded once to the
// tensors' type): the gradients of the query, the appended rows and the
// cache given those of the outputs (attention, context, and the returned
// caches).  The page "Autoregressive KV-cache append and causal attention"
// grades gradients too (its workspace note); the forward is the one of
// Required behavior, so with K', V' the
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
// Kernels: bwd_stats (one workgroup per (b, KV head, 64-slot chunk, row
// group): each packed row's max, sum and sum of P dP over the chunk's
// slots, K' and V' staged once for the group's rows), bwd_rows (one wave per packed
// row: the chunk statistics merged as the forward merges its segments),
// bwd_chunk (one workgroup per (b, KV head, 64-slot chunk): dS for the
// chunk's slots and all packed rows, the slot gradients, and per-chunk dq
// partials), bwd_dq (one wave per packed row: the partials summed).  The
// products of the two chunk kernels (scores, dO . V', dK', dV', dq) run on
// the fp64 matrix cores; the slot gradients are summed in fp64 and rounded
// once when stored.
#pragma once

#include "kvc_common.h"

namespace kvc {

constexpr int kBwdThreads = 256;
constexpr int kBwdSlots = 64;   // slots per chunk workgroup
constexpr int kBwdRowTile = 16;   // packed rows per tile in bwd_stats
// bwd_chunk takes 32 packed rows per tile (two 16-row blocks, independent
// product chains, half the barriers) when a head has more than 16, else 16
constexpr int kBwdChunkRowsWide = 32;
constexpr int kBwdMaxRowGroups = 16;

struct BwdArgs {
  int64_t B, Hq, Hk, Q, M, D, Dv;
  int32_t G, R;
  int64_t nchunk;  // partials per head: ceil(M / part_slots)
  int32_t part_slots;  // slots per partial (kBwdSlots here, kBwdVecSlots in kvc_backward_vec.h)
  int32_t gen_slots;  // kvc_backward_generic.h: slots per piece of a chunk
  int32_t row_groups;  // bwd_stats: workgroups per chunk, each over every row_groups-th row tile
  float scale;
  double scale_d;  // the same scale in fp64 (kvc_backward_generic.h)
  // tensors of the element type T the kernels are built for (float or bf16)
  const void* query;       // [B][Hq][Q][D]
  const void* new_key;     // [B][Hk][Q][D]
  const void* new_value;   // [B][Hk][Q][Dv]
  const void* kc;          // [B][Hk][M][D]: slots < length (the updated cache or the old one)
  const void* vc;
  const int64_t* lengths;  // the step's input lengths
  const uint8_t* mask;
  const void* d_att;       // gradients of the outputs (null = zero)
  const void* d_ctx;
  const void* d_kc_out;    // [B][Hk][M][D]
  const void* d_vc_out;
  void* g_query;           // gradients of the inputs
  void* g_new_key;
  void* g_new_value;
  void* g_kc;
  void* g_vc;
  double* ws_row;          // [B][Hq][Q][4]: m, l, sum_k P_k dP_k / l
  double* ws_part;         // [B*Hk][nchunk][R][4]: m_c, l_c, sum over the chunk of e^(s-m_c) dP
  double* ws_dq;           // [B*Hk][nchunk][R][D]
  float* ws_sdp;           // vector path: [B*Hk][R][M][2] score and dP of each visible slot
};

// Row information of batch row b: its length and prefix count n (0 for a
// row outside the contract).  Called by whole waves: lane t reads mask
// entry t of each 64-entry piece and the wave's ballot gives the prefix,
// so no load waits on another.
__device__ inline void bwd_row_info(const BwdArgs& a, int64_t b, int64_t* len, int64_t* n) {
  const int lane = threadIdx.x % kWave;
  const int64_t L = a.lengths[b];
  int64_t k = 0;
  bool open = true, ok = true;  // open: every entry so far is set
  for (int64_t base = 0; base < a.Q; base += kWave) {
    const int64_t t = base + lane;
    const uint64_t set = __ballot(t < a.Q && a.mask[b * a.Q + t] != 0);
    const int64_t cnt = a.Q - base < kWave ? a.Q - base : kWave;
    if (open) {
      const uint64_t all = cnt == kWave ? ~0ull : (1ull << cnt) - 1;
      if (set == all) {
        k += cnt;
      } else {  // entries [0, lead) set, entry lead clear: nothing above may be set
        const int lead = __builtin_ctzll(~set);
        k += lead;
        open = false;
        ok = (set >> lead) == 0;
      }
    } else {
      ok = ok && set == 0;
    }
  }
  ok = ok && L >= 0 && L <= a.M && L + k <= a.M;
  *len = L;
  *n = ok ? k : 0;
}

// Element access: values are widened exactly to fp32 as they are loaded,
// and each gradient is rounded once to the element type as it is stored.
template <typename T>
__device__ __forceinline__ float bwd_ld(const void* p, int64_t i) {
  if constexpr (sizeof(T) == 2)
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else
    return static_cast<const float*>(p)[i];
}
// Element i of p where ok, else 0.
//   fp32: masked-off lanes issue no load (the load sits in a branch whose
//   value is used after it, so the loads of a batch all go out first).
//   bf16: the same form would widen inside the branch and wait for each
//   load in turn; instead every lane loads, a masked-off one element i_safe
//   of the same tensor (a valid element next to what the other lanes
//   read), and a select zeroes it.
template <typename T>
__device__ __forceinline__ float bwd_ld_or0(bool ok, const void* p, int64_t i, int64_t i_safe) {
  if constexpr (sizeof(T) == 2) {
    const float v = bwd_ld<T>(p, ok ? i : i_safe);
    return ok ? v : 0.f;
  } else {
    float v = 0.f;
    if (ok) v = static_cast<const float*>(p)[i];
    return v;
  }
}
template <typename T>
__device__ __forceinline__ void bwd_st(void* p, int64_t i, float v) {
  if constexpr (sizeof(T) == 2)
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else
    static_cast<float*>(p)[i] = v;
}

// Slot j of the updated caches (element offset of its first value, and the
// tensor): kept rows from the cache, appended rows (j >= len) from
// new_key / new_value.
__device__ inline const void* bwd_key_src(const BwdArgs& a, int64_t grp, int64_t len, int64_t j,
                                          int64_t* off) {
  *off = j < len ? (grp * a.M + j) * a.D : (grp * a.Q + (j - len)) * a.D;
  return j < len ? a.kc : a.new_key;
}
__device__ inline const void* bwd_value_src(const BwdArgs& a, int64_t grp, int64_t len,
                                            int64_t j, int64_t* off) {
  *off = j < len ? (grp * a.M + j) * a.Dv : (grp * a.Q + (j - len)) * a.Dv;
  return j < len ? a.vc : a.new_value;
}

// The chunk kernels run their products on the fp64 matrix cores
// (v_mfma_f64_16x16x4_f64, fp32 inputs widened exactly).  Operand layout
// (wave64): lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and
// holds D[4 i + l / 16][l % 16] for i < 4.  A workgroup holds the K', V'
// rows of its chunk; the packed rows go through in tiles of 16, and wave w
// owns the chunk's slots [16 w, 16 w + 16).
typedef double bwd_f64x4 __attribute__((ext_vector_type(4)));

// LDS row pitches (in elements): the operand reads run down a column
// (16 rows x 4 columns, or 4 rows x 16 columns per instruction); these
// pitches keep such reads on distinct banks.
template <int N>
constexpr int bwd_pitch() {
  return N + 4;
}

// N consecutive elements of row `off` of a T tensor, widened to fp32, in
// 16-byte loads (the row and the tensor are 16-byte aligned; the host
// checks); ok = false gives zeros (the loads then read the same row, which
// the caller chooses valid).
template <typename T, int N>
__device__ __forceinline__ void bwd_row_slice(const void* src, int64_t off, bool ok, float (&x)[N]) {
  if constexpr (sizeof(T) == 2) {
    static_assert(N % 8 == 0, "slice");
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + off);
    uint4 w[N / 8];
#pragma unroll
    for (int u = 0; u < N / 8; u++) w[u] = p[u];
#pragma unroll
    for (int u = 0; u < N / 8; u++) {
      const uint32_t h[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        x[8 * u + 2 * e] = ok ? __uint_as_float(h[e] << 16) : 0.f;
        x[8 * u + 2 * e + 1] = ok ? __uint_as_float(h[e] & 0xffff0000u) : 0.f;
      }
    }
  } else {
    static_assert(N % 4 == 0, "slice");
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
    float4 w[N / 4];
#pragma unroll
    for (int u = 0; u < N / 4; u++) w[u] = p[u];
#pragma unroll
    for (int u = 0; u < N / 4; u++) {
      x[4 * u] = ok ? w[u].x : 0.f;
      x[4 * u + 1] = ok ? w[u].y : 0.f;
      x[4 * u + 2] = ok ? w[u].z : 0.f;
      x[4 * u + 3] = ok ? w[u].w : 0.f;
    }
  }
}

// K', V' rows of the chunk starting at slot s0 (zeros past nvis), in 16-byte
// pieces of slot rows.  Every load is issued before the first LDS store, so
// the loads overlap; slots past nvis read the last visible slot's row (nvis >
// s0 here) and a select zeroes them.
template <typename T, int D, int DV>
__device__ inline void bwd_stage_kv(const BwdArgs& a, int64_t grp, int64_t len, int64_t nvis,
                                    int64_t s0, float* k_s, float* v_s) {
  constexpr int C = kBwdSlots, KP = bwd_pitch<D>(), VP = bwd_pitch<DV>();
  constexpr int EP = 16 / static_cast<int>(sizeof(T));  // elements per piece
  constexpr int NPK = C * (D / EP) / kBwdThreads, NPV = C * (DV / EP) / kBwdThreads;
  static_assert(D % EP == 0 && DV % EP == 0 && C * (D / EP) % kBwdThreads == 0 &&
                    C * (DV / EP) % kBwdThreads == 0, "staging shape");
  const int tid = threadIdx.x;
  float kx[NPK][EP], vx[NPV][EP];
#pragma unroll
  for (int u = 0; u < NPK; u++) {
    const int p = tid + u * kBwdThreads, sl = p / (D / EP), col = (p % (D / EP)) * EP;
    const int64_t j = s0 + sl;
    int64_t off = 0;
    const void* src = bwd_key_src(a, grp, len, j < nvis ? j : nvis - 1, &off);
    bwd_row_slice<T, EP>(src, off + col, j < nvis, kx[u]);
  }
#pragma unroll
  for (int u = 0; u < NPV; u++) {
    const int p = tid + u * kBwdThreads, sl = p / (DV / EP), col = (p % (DV / EP)) * EP;
    const int64_t j = s0 + sl;
    int64_t off = 0;
    const void* src = bwd_value_src(a, grp, len, j < nvis ? j : nvis - 1, &off);
    bwd_row_slice<T, EP>(src, off + col, j < nvis, vx[u]);
  }
#pragma unroll
  for (int u = 0; u < NPK; u++) {
    const int p = tid + u * kBwdThreads;
    float* dst = k_s + (p / (D / EP)) * KP + (p % (D / EP)) * EP;
#pragma unroll
    for (int e = 0; e < EP; e++) dst[e] = kx[u][e];
  }
#pragma unroll
  for (int u = 0; u < NPV; u++) {
    const int p = tid + u * kBwdThreads;
    float* dst = v_s + (p / (DV / EP)) * VP + (p % (DV / EP)) * EP;
#pragma unroll
    for (int e = 0; e < EP; e++) dst[e] = vx[u][e];
  }
}

// The inputs of one tile of 16 packed rows, held in registers from their
// loads until the tile before has finished with LDS (so the loads of tile
// r + 1 are in flight while tile r computes): q and dO as raw 16-byte pieces
// of their rows (zeros for rows that are not valid; widened only when the
// tile is committed to LDS, so no load is waited for earlier), this lane's
// four attention-gradient entries (rows 4 i + l / 16 of the tile, its slot
// j; 0 where not visible), and for threads below 16 the row's m, l and
// sum P dP (bwd_chunk).
template <typename T, int D, int DV, int RT>
struct BwdTileRegs {
  static constexpr int EP = 16 / static_cast<int>(sizeof(T));  // elements per piece
  static constexpr int PQ = RT * D / EP, PO = RT * DV / EP;     // pieces per tile
  static constexpr int NQ = (PQ + kBwdThreads - 1) / kBwdThreads;
  static constexpr int NO = (PO + kBwdThreads - 1) / kBwdThreads;
  static_assert(D % EP == 0 && DV % EP == 0, "row pieces");
  uint4 q[NQ], o[NO];
  float da[RT / 4];  // [16-row block][i]
  double st[3];
};

template <typename T, int D, int DV, int RT>
__device__ inline void bwd_fetch_tile(const BwdArgs& a, int64_t b, int64_t kvh, int64_t len,
                                      int64_t n, int r0, int64_t j, bool stats,
                                      BwdTileRegs<T, D, DV, RT>& x) {
  using X = BwdTileRegs<T, D, DV, RT>;
  constexpr int EP = X::EP;
  const int tid = threadIdx.x, lq = (tid % kWave) / 16;
  const int Q = static_cast<int>(a.Q);
  // the head's packed row r as a (b, query head, token) row; rows past R
  // (tile padding) read the head's last row instead
  auto qrow = [&](int r) {
    const int rc = r < a.R ? r : a.R - 1;
    return (b * a.Hq + kvh * a.G + rc / Q) * a.Q + rc % Q;
  };
  // q and dO pieces: a piece of a row that is not valid is not loaded
#pragma unroll
  for (int u = 0; u < X::NQ; u++) {
    const int p = tid + u * kBwdThreads, r = r0 + p / (D / EP);
    x.q[u] = uint4{0u, 0u, 0u, 0u};
    if (p < X::PQ && r < a.R && r % Q < n)
      x.q[u] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.query) + qrow(r) * D +
                                               (p % (D / EP)) * EP);
  }
#pragma unroll
  for (int u = 0; u < X::NO; u++) {
    const int p = tid + u * kBwdThreads, r = r0 + p / (DV / EP);
    x.o[u] = uint4{0u, 0u, 0u, 0u};
    if (a.d_ctx && p < X::PO && r < a.R && r % Q < n)
      x.o[u] = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.d_ctx) + qrow(r) * DV +
                                               (p % (DV / EP)) * EP);
  }
  if constexpr (sizeof(T) == 4) {  // masked-off lanes load nothing (see bwd_ld_or0)
#pragma unroll
    for (int k = 0; k < RT / 4; k++) {
      const int r = r0 + 16 * (k / 4) + 4 * (k % 4) + lq;
      const int g = r / Q, t = r % Q;
      const bool vis = a.d_att && r < a.R && t < n && j <= len + t;
      x.da[k] = vis ? bwd_ld<T>(a.d_att, ((b * a.Hq + kvh * a.G + g) * a.Q + t) * a.M + j) : 0.f;
    }
  } else {
#pragma unroll
  for (int k = 0; k < RT / 4; k++) x.da[k] = 0.f;
  if (a.d_att) {
    const int64_t jc = j < a.M ? j : a.M - 1;
#pragma unroll
    for (int k = 0; k < RT / 4; k++) {
      // rows grow with k: from the first group of four that is all tile
      // padding on, nothing is visible (the entries stay 0)
      if (r0 + 16 * (k / 4) + 4 * (k % 4) >= a.R) break;
      const int r = r0 + 16 * (k / 4) + 4 * (k % 4) + lq;
      const int t = r % Q;
      const bool vis = r < a.R && t < n && j <= len + t;
      x.da[k] = bwd_ld_or0<T>(vis, a.d_att, qrow(r) * a.M + j, qrow(r) * a.M + jc);
    }
  }
  }
  if (stats && tid < RT) {
    const int r = r0 + tid;
    const bool ok = r < a.R && r % Q < n;
    const double* st = a.ws_row + qrow(r) * 4;
    x.st[0] = ok ? st[0] : 0.0;
    x.st[1] = ok ? st[1] : 1.0;
    x.st[2] = ok ? st[2] : 0.0;
  }
}

// 16-byte piece w of a T row, widened to fp32.
template <typename T>
__device__ __forceinline__ void bwd_widen(const uint4& w, float (&v)[16 / sizeof(T)]) {
  const uint32_t h[4] = {w.x, w.y, w.z, w.w};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int k = 0; k < 4; k++) {  // little-endian: element 2k in the low half
      v[2 * k] = __uint_as_float(h[k] << 16);
      v[2 * k + 1] = __uint_as_float(h[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = __uint_as_float(h[k]);
  }
}

// q and dO of the tile into LDS (row pitches KP and VP elements).
template <typename T, int D, int DV, int RT, int KP = bwd_pitch<D>(), int VP = bwd_pitch<DV>()>
__device__ inline void bwd_commit_tile(const BwdTileRegs<T, D, DV, RT>& x, float* q_s,
                                       float* o_s) {
  using X = BwdTileRegs<T, D, DV, RT>;
  constexpr int EP = X::EP;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < X::NQ; u++) {
    const int p = tid + u * kBwdThreads;
    if (p < X::PQ) {
      float v[EP];
      bwd_widen<T>(x.q[u], v);
      float* dst = q_s + (p / (D / EP)) * KP + (p % (D / EP)) * EP;
#pragma unroll
      for (int e = 0; e < EP; e++) dst[e] = v[e];
    }
  }
#pragma unroll
  for (int u = 0; u < X::NO; u++) {
    const int p = tid + u * kBwdThreads;
    if (p < X::PO) {
      float v[EP];
      bwd_widen<T>(x.o[u], v);
      float* dst = o_s + (p / (DV / EP)) * VP + (p % (DV / EP)) * EP;
#pragma unroll
      for (int e = 0; e < EP; e++) dst[e] = v[e];
    }
  }
}

// S = q . K'_j and dO . V'_j for the 16 staged rows and this wave's 16
// slots: s[i], dov[i] belong to row 4 i + l / 16 and slot 16 w + l % 16.
template <int D, int DV>
__device__ inline void bwd_scores(const float* q_s, const float* o_s, const float* k_s,
                                  const float* v_s, int w, int li, int lq, bwd_f64x4& s,
                                  bwd_f64x4& dov) {
  constexpr int KP = bwd_pitch<D>(), VP = bwd_pitch<DV>();
  s = bwd_f64x4{0.0, 0.0, 0.0, 0.0};
  dov = bwd_f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int kk = 0; kk < D / 4; kk++)
    s = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(q_s[li * KP + 4 * kk + lq]),
                                             static_cast<double>(k_s[(16 * w + li) * KP + 4 * kk + lq]),
                                             s, 0, 0, 0);
#pragma unroll
  for (int kk = 0; kk < DV / 4; kk++)
    dov = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(o_s[li * VP + 4 * kk + lq]),
                                               static_cast<double>(v_s[(16 * w + li) * VP + 4 * kk + lq]),
                                               dov, 0, 0, 0);
}


// One workgroup per (b, KV head, chunk of kBwdSlots slots, row group): for
// every valid packed row of its row tiles, over the chunk's slots it sees, m_c = max s_j, l_c =
// sum e^(s_j - m_c) and sum e^(s_j - m_c) dP_j, in fp64 (each wave over its
// 16 slots, then the four merged).  Held to two waves per SIMD: at D = 128
// the compiler otherwise takes 262 registers and runs one.
template <typename T, int D, int DV>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void
bwd_stats_kernel(BwdArgs a) {
  constexpr int C = kBwdSlots, RT = kBwdRowTile, W = kBwdThreads / kWave;
  // The products run over the head dimension in the order where lane group
  // l / 16 takes the contiguous quarter [lq D/4, (lq + 1) D/4): so each
  // lane's K' (and V') operands are one contiguous slice of its slot's row,
  // loaded straight into registers, and only the q and dO tiles go through
  // LDS (odd pitches: the A-operand reads hit distinct banks).
  constexpr int KQ = D / 4, VQ = DV / 4, QP = D + 1, OP = DV + 1;
  static_assert(C == 16 * W && RT == 16 && D % 32 == 0 && DV % 32 == 0, "tile shape");
  __shared__ float q_s[RT * QP];
  __shared__ float o_s[RT * OP];
  __shared__ double part_s[W][RT][3];
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane % 16, lq = lane / 16;
  const int rg = static_cast<int>(blockIdx.x % a.row_groups);
  const int64_t c = (blockIdx.x / a.row_groups) % a.nchunk;
  const int64_t grp = blockIdx.x / a.row_groups / a.nchunk;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  const int64_t s0 = c * C;
  const int64_t nvis = n > 0 ? len + n : 0;
  if (s0 >= nvis || rg * RT >= a.R) return;  // no row of this workgroup sees the chunk
  const double scale = a.scale;
  const int64_t j = s0 + 16 * wave + li;  // this lane's slot
  const int step = a.row_groups * RT;
  BwdTileRegs<T, D, DV, RT> nx;  // the next tile's inputs, loading while this one computes
  bwd_fetch_tile<T, D, DV, RT>(a, b, kvh, len, n, rg * RT, j, false, nx);
  // this lane's K' and V' operand slices (slots past nvis: zeros, read from
  // the last visible slot's row, nvis > s0 here)
  float kx[KQ], vx[VQ];
  {
    const int64_t jr = j < nvis ? j : nvis - 1;
    int64_t koff = 0, voff = 0;
    const void* ksrc = bwd_key_src(a, grp, len, jr, &koff);
    const void* vsrc = bwd_value_src(a, grp, len, jr, &voff);
    bwd_row_slice<T, KQ>(ksrc, koff + lq * KQ, j < nvis, kx);
    bwd_row_slice<T, VQ>(vsrc, voff + lq * VQ, j < nvis, vx);
  }
  for (int r0 = rg * RT; r0 < a.R; r0 += step) {
    __syncthreads();  // the previous tile is no longer read
    bwd_commit_tile<T, D, DV, RT, QP, OP>(nx, q_s, o_s);
    float da[4];
#pragma unroll
    for (int i = 0; i < 4; i++) da[i] = nx.da[i];
    __syncthreads();
    if (r0 + step < a.R) bwd_fetch_tile<T, D, DV, RT>(a, b, kvh, len, n, r0 + step, j, false, nx);
    bwd_f64x4 s = {0.0, 0.0, 0.0, 0.0}, dov = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kk = 0; kk < KQ; kk++)
      s = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(q_s[li * QP + lq * KQ + kk]),
                                               static_cast<double>(kx[kk]), s, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < VQ; kk++)
      dov = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(o_s[li * OP + lq * VQ + kk]),
                                                 static_cast<double>(vx[kk]), dov, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      // rows grow with i: groups of four that are all tile padding are not
      // reduced (the merge below reads rows below R only)
      if (r0 + 4 * i >= a.R) break;
      const int r = r0 + 4 * i + lq;
      const int t = r % static_cast<int>(a.Q);
      const bool vis = r < a.R && t < n && j <= len + t;
      const double sc = scale * s[i];
      const double dp = vis ? dov[i] + static_cast<double>(da[i]) : 0.0;
      double m = vis ? sc : -INFINITY;
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const double y = __shfl_xor(m, o);
        m = y > m ? y : m;
      }
      const double e = vis ? exp(sc - m) : 0.0;
      double l = e, pd = e * dp;
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        l += __shfl_xor(l, o);
        pd += __shfl_xor(pd, o);
      }
      if (li == 0) {
        part_s[wave][4 * i + lq][0] = m;
        part_s[wave][4 * i + lq][1] = l;
        part_s[wave][4 * i + lq][2] = pd;
      }
    }
    __syncthreads();
    if (tid < RT) {  // the four strips of each row merged
      const int r = r0 + tid;
      const int t = r % static_cast<int>(a.Q);
      if (r < a.R && t < n) {
        double m = -INFINITY, l = 0, pd = 0;
#pragma unroll
        for (int w = 0; w < W; w++) m = part_s[w][tid][0] > m ? part_s[w][tid][0] : m;
#pragma unroll
        for (int w = 0; w < W; w++) {
          const double mw = part_s[w][tid][0];
          const double f = mw == -INFINITY ? 0.0 : exp(mw - m);
          l += part_s[w][tid][1] * f;
          pd += part_s[w][tid][2] * f;
        }
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
  const int64_t nc = t < n ? (len + t) / a.part_slots + 1 : 0;
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

// Piece p (16 bytes, slot p / (N / EP), elements from (p % (N / EP)) EP on)
// of a chunk's slot rows of the pass-through gradient src [B, Hk, M, N]:
// zeros for a NULL src and past M.  Every lane loads (slots past M read the
// last slot's row) and a select zeroes, so no load waits inside a branch.
template <typename T, int N>
__device__ __forceinline__ uint4 bwd_pass_piece(const BwdArgs& a, const void* src, int64_t grp,
                                                int64_t s0, int p) {
  constexpr int EP = 16 / static_cast<int>(sizeof(T)), PR = N / EP;
  if (!src) return uint4{0u, 0u, 0u, 0u};
  const int64_t js = s0 + p / PR, jc = js < a.M ? js : a.M - 1;
  const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const T*>(src) +
                                                  (grp * a.M + jc) * N + (p % PR) * EP);
  return js < a.M ? x : uint4{0u, 0u, 0u, 0u};
}

// Piece p of the chunk's slot gradients: the pass-through x plus the
// products' part from the LDS tile (pitch TP floats), rounded once to T.
// Kept slots -> g_cache; appended ones (len <= j < len + n) -> their row of
// g_new, with zeros in g_cache; nothing past M.
template <typename T, int N, int TP>
__device__ __forceinline__ void bwd_piece_out(const BwdArgs& a, int64_t grp, int64_t len,
                                              int64_t n, int64_t s0, int p, const uint4& x,
                                              const float* tile, void* g_cache, void* g_new) {
  constexpr int EP = 16 / static_cast<int>(sizeof(T)), PR = N / EP;
  const int sl = p / PR, col = (p % PR) * EP;
  const int64_t js = s0 + sl;
  if (js >= a.M) return;
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  float v[EP];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int k = 0; k < 4; k++) {  // little-endian: element 2k in the low half
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = __uint_as_float(w[k]);
  }
  const float* t = tile + sl * TP + col;
#pragma unroll
  for (int e = 0; e < EP; e++) v[e] = t[e] + v[e];
  uint32_t y[4];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int k = 0; k < 4; k++)
      y[k] = static_cast<uint32_t>(f32_to_bf16(v[2 * k])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * k + 1])) << 16);
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) y[k] = __float_as_uint(v[k]);
  }
  const uint4 out{y[0], y[1], y[2], y[3]};
  uint4* at = reinterpret_cast<uint4*>(static_cast<T*>(g_cache) + (grp * a.M + js) * N + col);
  if (js >= len && js < len + n) {
    *reinterpret_cast<uint4*>(static_cast<T*>(g_new) + (grp * a.Q + (js - len)) * N + col) = out;
    *at = uint4{0u, 0u, 0u, 0u};
  } else {
    *at = out;
  }
}

// One workgroup per (b, KV head, chunk of kBwdSlots slots, column group):
// dS for the chunk's slots and every packed row, and for the group's
// columns the slot gradients of the chunk and the chunk's share of every
// row's dq.
template <typename T, int D, int DV, int RT>
__global__ __launch_bounds__(kBwdThreads) void bwd_chunk_kernel(BwdArgs a) {
  constexpr int C = kBwdSlots, NB = RT / 16, W = kBwdThreads / kWave;
  constexpr int KP = bwd_pitch<D>(), VP = bwd_pitch<DV>(), SP = C + 1;
  constexpr int DT = D / 16, VT = DV / 16;  // 16-column tiles of dK'/dq and dV'
  static_assert(C == 16 * W && RT % 16 == 0 && D % 16 == 0 && DV % 16 == 0, "tile shape");
  __shared__ float k_s[C * KP];
  __shared__ float v_s[C * VP];
  __shared__ float q_s[RT * KP];
  __shared__ float o_s[RT * VP];
  __shared__ double ds_s[RT * SP];  // scale * dS (0 where not visible)
  __shared__ double p_s[RT * SP];   // P (0 where not visible)
  __shared__ double st_s[RT][3];    // the rows' m, l and sum_k P_k dP_k
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int li = lane % 16, lq = lane / 16;
  const int64_t c = blockIdx.x % a.nchunk;
  const int64_t grp = blockIdx.x / a.nchunk;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  const int64_t s0 = c * C;
  constexpr int dc0 = 0, vc0 = 0;  // first dK'/dq and dV' column
  // slots with any attention gradient (none on a row that appends nothing
  // or is rejected; then only the pass-through below remains)
  const int64_t nvis = n > 0 ? len + n : 0;
  const bool any = s0 < nvis;  // nvis <= M
  const int64_t j = s0 + 16 * wave + li;  // this lane's slot in the score tile
  BwdTileRegs<T, D, DV, RT> nx;  // the next tile's inputs, loading while this one computes
  if (any) {
    bwd_fetch_tile<T, D, DV, RT>(a, b, kvh, len, n, 0, j, true, nx);
    bwd_stage_kv<T, D, DV>(a, grp, len, nvis, s0, k_s, v_s);
  }

  // dK', dV' of this wave's 16 slots: gk[dt][i] = dK'[slot 16 w + 4 i + lq][dc0 + 16 dt + li]
  bwd_f64x4 gk[DT], gv[VT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) gk[dt] = bwd_f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int vt = 0; vt < VT; vt++) gv[vt] = bwd_f64x4{0.0, 0.0, 0.0, 0.0};

  const double scale = a.scale;
  for (int r0 = 0; any && r0 < a.R; r0 += RT) {
    __syncthreads();  // the previous tile is no longer read
    bwd_commit_tile<T, D, DV, RT>(nx, q_s, o_s);
    if (tid < RT) {
      st_s[tid][0] = nx.st[0];
      st_s[tid][1] = nx.st[1];
      st_s[tid][2] = nx.st[2];
    }
    float da[RT / 4];
#pragma unroll
    for (int k = 0; k < RT / 4; k++) da[k] = nx.da[k];
    __syncthreads();
    if (r0 + RT < a.R) bwd_fetch_tile<T, D, DV, RT>(a, b, kvh, len, n, r0 + RT, j, true, nx);
    // P from the score and the row's m, l; dS = P (dP - sum_k P_k dP_k);
    // the 16-row blocks' products are independent chains
    bwd_f64x4 s[NB], dov[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++)
      bwd_scores<D, DV>(q_s + nb * 16 * KP, o_s + nb * 16 * VP, k_s, v_s, wave, li, lq, s[nb],
                        dov[nb]);
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int rr = 16 * nb + 4 * i + lq, r = r0 + rr;
        const int t = r % static_cast<int>(a.Q);
        const bool vis = r < a.R && t < n && j <= len + t;
        double p = 0.0, ds = 0.0;
        if (vis) {
          const double dp = dov[nb][i] + static_cast<double>(da[4 * nb + i]);
          p = exp(scale * s[nb][i] - st_s[rr][0]) / st_s[rr][1];
          ds = scale * p * (dp - st_s[rr][2]);
        }
        ds_s[rr * SP + 16 * wave + li] = ds;
        p_s[rr * SP + 16 * wave + li] = p;
      }
    }
    __syncthreads();  // dq below reads every wave's slots
    // dK'_j += sum_r scale dS q_r and dV'_j += sum_r P dO_r over the tile's rows
    // (groups of 4 rows; groups past the head's last packed row are padding)
#pragma unroll
    for (int kk = 0; kk < RT / 4; kk++) {
      if (r0 + 4 * kk >= a.R) break;
      const double dsa = ds_s[(4 * kk + lq) * SP + 16 * wave + li];
      const double pa = p_s[(4 * kk + lq) * SP + 16 * wave + li];
#pragma unroll
      for (int dt = 0; dt < DT; dt++)
        gk[dt] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            dsa, static_cast<double>(q_s[(4 * kk + lq) * KP + dc0 + 16 * dt + li]), gk[dt], 0, 0, 0);
#pragma unroll
      for (int vt = 0; vt < VT; vt++)
        gv[vt] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            pa, static_cast<double>(o_s[(4 * kk + lq) * VP + vc0 + 16 * vt + li]), gv[vt], 0, 0, 0);
    }
    // the chunk's share of dq = sum_j scale dS_j K'_j over this workgroup's
    // columns: wave w takes its 16-column tiles w, w + W, ...
    for (int dt = wave; dt < DT; dt += W) {
      bwd_f64x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; nb++) acc[nb] = bwd_f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int kk = 0; kk < C / 4; kk++) {
        const double kb = static_cast<double>(k_s[(4 * kk + lq) * KP + dc0 + 16 * dt + li]);
#pragma unroll
        for (int nb = 0; nb < NB; nb++)
          acc[nb] = __builtin_amdgcn_mfma_f64_16x16x4f64(ds_s[(16 * nb + li) * SP + 4 * kk + lq],
                                                         kb, acc[nb], 0, 0, 0);
      }
#pragma unroll
      for (int nb = 0; nb < NB; nb++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int r = r0 + 16 * nb + 4 * i + lq;
          if (r < a.R)
            a.ws_dq[((grp * a.nchunk + c) * a.R + r) * D + dc0 + 16 * dt + li] = acc[nb][i];
        }
      }
    }
  }

  // Slot gradients out, in 16-byte pieces of slot rows: each wave's dK'/dV'
  // strip goes through LDS (the K'/V' tiles are no longer read), so that a
  // thread adds the pass-through to whole pieces and stores them with one
  // instruction each.  All pass-through pieces are loaded before the first
  // store: the host refuses overlapping buffers, but the compiler cannot
  // know that and would otherwise wait for each load in turn.
  constexpr int EP = 16 / static_cast<int>(sizeof(T));  // elements per piece
  constexpr int NPK = C * (D / EP) / kBwdThreads, NPV = C * (DV / EP) / kBwdThreads;
  static_assert(D % EP == 0 && DV % EP == 0 && C * (D / EP) % kBwdThreads == 0 &&
                    C * (DV / EP) % kBwdThreads == 0, "piece shape");
  __syncthreads();  // every wave is past its last read of k_s / v_s
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int sl = 16 * wave + 4 * i + lq;
#pragma unroll
    for (int dt = 0; dt < DT; dt++) k_s[sl * KP + 16 * dt + li] = static_cast<float>(gk[dt][i]);
#pragma unroll
    for (int vt = 0; vt < VT; vt++) v_s[sl * VP + 16 * vt + li] = static_cast<float>(gv[vt][i]);
  }
  uint4 xk[NPK], xv[NPV];
#pragma unroll
  for (int u = 0; u < NPK; u++)
    xk[u] = bwd_pass_piece<T, D>(a, a.d_kc_out, grp, s0, tid + u * kBwdThreads);
#pragma unroll
  for (int u = 0; u < NPV; u++)
    xv[u] = bwd_pass_piece<T, DV>(a, a.d_vc_out, grp, s0, tid + u * kBwdThreads);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NPK; u++)
    bwd_piece_out<T, D, KP>(a, grp, len, n, s0, tid + u * kBwdThreads, xk[u], k_s, a.g_kc,
                            a.g_new_key);
#pragma unroll
  for (int u = 0; u < NPV; u++)
    bwd_piece_out<T, DV, VP>(a, grp, len, n, s0, tid + u * kBwdThreads, xv[u], v_s, a.g_vc,
                             a.g_new_value);
  // appended rows that do not exist (t >= n, rejected rows): zero gradient
  if (c == 0) {
    for (int64_t idx = tid; idx < (a.Q - n) * D; idx += kBwdThreads)
      bwd_st<T>(a.g_new_key, (grp * a.Q + n + idx / D) * D + idx % D, 0.f);
    for (int64_t idx = tid; idx < (a.Q - n) * DV; idx += kBwdThreads)
      bwd_st<T>(a.g_new_value, (grp * a.Q + n + idx / DV) * DV + idx % DV, 0.f);
  }
}

// dq_r = sum over the chunks its row can see of the partials (0 for rows
// that are not valid).  One workgroup per row: thread (cl, d) sums column d
// over the chunks cl, cl + CL, ... (CL = kBwdThreads / D column lanes, four
// independent sums so that several loads are in flight), then the CL sums
// are merged in LDS.  D divides kBwdThreads (the host admits D in {64, 128}).
template <typename T>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(BwdArgs a) {
  __shared__ double part_s[kBwdThreads];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int D = static_cast<int>(a.D), CL = kBwdThreads / D, cl = tid / D, d = tid % D;
  const int64_t t = row % a.Q, hq = (row / a.Q) % a.Hq, b = row / (a.Hq * a.Q);
  int64_t len, n;
  bwd_row_info(a, b, &len, &n);
  const int64_t kvh = hq / a.G, g = hq % a.G, r = g * a.Q + t, grp = b * a.Hk + kvh;
  const int64_t nc = t < n ? (len + t) / a.part_slots + 1 : 0;  // partials over slots <= len + t
  const int64_t cs = static_cast<int64_t>(a.R) * D;          // one chunk's stride
  const double* p = a.ws_dq + (grp * a.nchunk * a.R + r) * D + d;
  double s0 = 0, s1 = 0, s2 = 0, s3 = 0;
  int64_t c = cl;
  for (; c + 3 * CL < nc; c += 4 * CL) {
    s0 += p[c * cs];
    s1 += p[(c + CL) * cs];
    s2 += p[(c + 2 * CL) * cs];
    s3 += p[(c + 3 * CL) * cs];
  }
  for (; c < nc; c += CL) s0 += p[c * cs];
  part_s[tid] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  if (tid < D) {
    double acc = 0;
    for (int k = 0; k < CL; k++) acc += part_s[k * D + tid];
    bwd_st<T>(a.g_query, row * D + tid, static_cast<float>(acc));
  }
}

}  // namespace kvc
