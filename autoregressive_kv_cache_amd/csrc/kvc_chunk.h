// kvc_chunk.h -- attend kernel for many packed query rows per KV head
// (multi-token appends: G * Q > 8), bf16, on the matrix cores.
//
// One workgroup handles one (batch row b, KV head h, chunk c of 64 slots)
// and one group of up to 64 packed query rows of that head (row r = g * Q +
// t reads query head h * G + g, token t; chunk_row_groups groups per chunk):
//   1. (first group only) cache writes for the chunk's slot range, as on the page
//      "Autoregressive KV-cache append and causal attention" (Required
//      behavior): new rows at slot length + t, out of place every other slot
//      copied bit for bit;
//   2. the chunk's K rows [64 x D] into LDS and its V rows transposed
//      [Dv x 64] into LDS (the appended slots read from new_key/new_value,
//      slots past length + n as zeros), shared by the four waves;
//   3. per block of 16 packed rows (one wave): S = Q K^T with
//      v_mfma_f32_16x16x32_bf16 (fp32 accumulation), scale, the causal mask
//      j <= length + t (lower-right alignment, KempnerForge PR 542), the
//      chunk statistics m_c = max s_j and l_c = sum exp(s_j - m_c), the
//      values exp(s_j - m_c) into the attention buffer, and
//      o_c = sum_j exp(s_j - m_c) v_j with a second matrix product.
// Every chunk is its own segment (dense mode); the combine kernel merges
// them exactly as it merges the other attend kernels' results.
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies
// A[l % 16][8 * (l / 16) + e] and B[8 * (l / 16) + e][l % 16] for e < 8, and
// receives D[4 * (l / 16) + i][l % 16] for i < 4.
#pragma once

#include "kvc_common.h"
#include "kvc_generic.h"

namespace kvc {

constexpr int kChunkSlots = 64;      // slots per chunk (C)
constexpr int kChunkThreads = 256;   // four waves
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kChunkBlockRows = 16;  // packed rows per matrix block

// Workgroups per (b, KV head, chunk): each takes kChunkWaves blocks of 16
// packed rows (one per wave), so many packed rows spread over more compute
// units instead of queueing on one.
__host__ __device__ inline int chunk_row_groups(int64_t R) {
  const int64_t nblk = (R + kChunkBlockRows - 1) / kChunkBlockRows;
  const int64_t g = (nblk + kChunkWaves - 1) / kChunkWaves;
  return static_cast<int>(g > 0 ? g : 1);
}

typedef __bf16 mfma_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mfma_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ mfma_f32x4 mfma_16x16x32(const uint4& a, const uint4& b,
                                                    mfma_f32x4 c) {
  mfma_bf16x8 av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint4 ld_lds16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

template <int D, int DV>
__global__ __launch_bounds__(kChunkThreads) void attend_chunk_kernel(StepArgs a) {
  constexpr int C = kChunkSlots;
  constexpr int KP = D + 8;   // K row pitch in LDS (elements; 16-byte multiple)
  constexpr int VP = C + 8;   // V^T row pitch
  constexpr int PP = C + 8;   // probability tile pitch
  static_assert(D % 32 == 0 && DV % 16 == 0, "head sizes");
  __shared__ __align__(16) uint16_t k_s[C * KP];
  __shared__ __align__(16) uint16_t vt_s[DV * VP];
  __shared__ __align__(16) uint16_t p_s[kChunkWaves][kChunkBlockRows * PP];
  __shared__ RowInfo info_sh;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int RG = chunk_row_groups(a.R);
  const int rg = static_cast<int>(blockIdx.x % RG);
  const int64_t c = (blockIdx.x / RG) % a.nchunk_max;
  const int64_t grp = blockIdx.x / RG / a.nchunk_max;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;

  if (wave == 0) {
    const RowInfo ri = wave_row_info(a.lengths, a.mask, a.Q, a.M, b);
    if (lane == 0) info_sh = ri;
  }
  __syncthreads();
  const RowInfo ri = info_sh;
  if (c == 0 && kvh == 0 && rg == 0 && tid == 0) {
    a.ws_rowinfo[b * 4 + 0] = ri.len;
    a.ws_rowinfo[b * 4 + 1] = ri.n;
    a.ws_rowinfo[b * 4 + 2] = ri.status;
    a.ws_rowinfo[b * 4 + 3] = 0;
  }
  const int64_t len = ri.len, n = ri.n, new_len = len + n;
  const int64_t s0 = c * C;
  const int64_t s1 = s0 + C < a.M ? s0 + C : a.M;

  const int64_t head = b * a.Hk + kvh;
  // slot j of the head at k_head + j * D: the dense cache, or (paged) the
  // chunk's block, which holds all of its slots; null = outside the pool
  const uint16_t* k_head = static_cast<const uint16_t*>(a.kc_in) + head * a.M * D;
  const uint16_t* v_head = static_cast<const uint16_t*>(a.vc_in) + head * a.M * DV;
  if (a.paged) {
    const auto* kp = reinterpret_cast<const uint16_t*>(slot_row(a, a.kc_in, b, kvh, s0, D * 2));
    const auto* vp = reinterpret_cast<const uint16_t*>(slot_row(a, a.vc_in, b, kvh, s0, DV * 2));
    k_head = kp ? kp - s0 * D : nullptr;
    v_head = vp ? vp - s0 * DV : nullptr;
  }
  const uint16_t* nk_head = static_cast<const uint16_t*>(a.new_key) + head * a.Q * D;
  const uint16_t* nv_head = static_cast<const uint16_t*>(a.new_value) + head * a.Q * DV;

  // 1. cache writes of the slot range [s0, s1)
  if (rg == 0 && !a.read_only) {  // the chunk's cache writes, once
    // (paged: in place, into the chunk's block, which is the one read)
    uint8_t* kd = a.paged ? const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(k_head))
                          : static_cast<uint8_t*>(a.kc_out) + head * a.M * D * 2;
    uint8_t* vd = a.paged ? const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(v_head))
                          : static_cast<uint8_t*>(a.vc_out) + head * a.M * DV * 2;
    if (kd)
      write_cache_slots(kd, reinterpret_cast<const uint8_t*>(k_head),
                        reinterpret_cast<const uint8_t*>(nk_head), D * 2, s0, s1, len, n,
                        a.out_of_place != 0, tid, kChunkThreads);
    if (vd)
      write_cache_slots(vd, reinterpret_cast<const uint8_t*>(v_head),
                        reinterpret_cast<const uint8_t*>(nv_head), DV * 2, s0, s1, len, n,
                        a.out_of_place != 0, tid, kChunkThreads);
  }
  if (a.R == 0 || c >= row_chunks(len, n, C)) return;
  const int nact = static_cast<int>((s1 < new_len ? s1 : new_len) - s0);  // visited slots

  // 2. K rows and transposed V rows of the chunk into LDS.  Every 16-byte
  // load is issued before the first LDS store, so the loads overlap.
  constexpr int NK = C * (D / 8) / kChunkThreads, NV = C * (DV / 8) / kChunkThreads;
  static_assert(NK * kChunkThreads == C * (D / 8) && NV * kChunkThreads == C * (DV / 8),
                "staging shape");
  uint4 kx[NK], vx[NV];
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int idx = tid + i * kChunkThreads, slot = idx / (D / 8), part = idx % (D / 8);
    const int64_t j = s0 + slot;
    kx[i] = make_uint4(0, 0, 0, 0);
    if (slot < nact && (j >= len || k_head))
      kx[i] = ld_global16((j < len ? k_head + j * D : nk_head + (j - len) * D) + part * 8);
  }
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int idx = tid + i * kChunkThreads, slot = idx % C, part = idx / C;
    const int64_t j = s0 + slot;
    vx[i] = make_uint4(0, 0, 0, 0);
    if (slot < nact && (j >= len || v_head))
      vx[i] = ld_global16((j < len ? v_head + j * DV : nv_head + (j - len) * DV) + part * 8);
  }
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int idx = tid + i * kChunkThreads, slot = idx / (D / 8), part = idx % (D / 8);
    *reinterpret_cast<uint4*>(k_s + slot * KP + part * 8) = kx[i];
  }
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int idx = tid + i * kChunkThreads, slot = idx % C, part = idx / C;
    const uint32_t w[4] = {vx[i].x, vx[i].y, vx[i].z, vx[i].w};
#pragma unroll
    for (int e = 0; e < 4; e++) {
      vt_s[(part * 8 + 2 * e) * VP + slot] = static_cast<uint16_t>(w[e] & 0xffffu);
      vt_s[(part * 8 + 2 * e + 1) * VP + slot] = static_cast<uint16_t>(w[e] >> 16);
    }
  }
  __syncthreads();

  // 3. blocks of 16 packed rows, one wave each
  const float scale = static_cast<float>(a.scale);
  const float neg_inf = -INFINITY;
  const int li = lane % 16, lq = lane / 16;
  const int64_t seg = grp * a.nchunk_max + c;
  const uint16_t* qbase = static_cast<const uint16_t*>(a.query);
  uint16_t* att = static_cast<uint16_t*>(a.attention);
  uint16_t* ptile = p_s[wave];
  const int nblk = (a.R + kChunkBlockRows - 1) / kChunkBlockRows;
  const int blk_end = (rg + 1) * kChunkWaves < nblk ? (rg + 1) * kChunkWaves : nblk;
  for (int blk = rg * kChunkWaves + wave; blk < blk_end; blk += kChunkWaves) {
    // query rows as A operands: lane holds row li, dims kk*32 + 8*lq + e
    uint4 qa[D / 32];
    {
      const int r = blk * kChunkBlockRows + li;
      const int64_t g = r / a.Q, t = r % a.Q;
      const bool ok = r < a.R && t < n;
      const uint16_t* qrow = qbase + ((b * a.Hq + kvh * a.G + g) * a.Q + t) * D;
#pragma unroll
      for (int kk = 0; kk < D / 32; kk++)
        qa[kk] = ok ? ld_global16(qrow + kk * 32 + 8 * lq) : make_uint4(0, 0, 0, 0);
    }
    // scores: s[jt][i] = S[4*lq + i][jt*16 + li]
    mfma_f32x4 s[C / 16];
#pragma unroll
    for (int jt = 0; jt < C / 16; jt++) {
      s[jt] = mfma_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; kk++)
        s[jt] = mfma_16x16x32(qa[kk], ld_lds16(k_s + (jt * 16 + li) * KP + kk * 32 + 8 * lq),
                              s[jt]);
    }
    // rows of this lane's outputs: packed rows blk*16 + 4*lq + i
    int64_t t_of[4];
    bool row_ok[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = blk * kChunkBlockRows + 4 * lq + i;
      t_of[i] = r % a.Q;
      row_ok[i] = r < a.R && t_of[i] < n;
    }
    float sv[C / 16][4];
#pragma unroll
    for (int jt = 0; jt < C / 16; jt++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int jl = jt * 16 + li;
        const bool ok = row_ok[i] && jl < nact && s0 + jl <= len + t_of[i];
        sv[jt][i] = ok ? s[jt][i] * scale : neg_inf;
      }
    // chunk statistics per row: over the 4 column tiles, then the 16 lanes
    // that share lq
    float m[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float x = sv[0][i];
#pragma unroll
      for (int jt = 1; jt < C / 16; jt++) x = sv[jt][i] > x ? sv[jt][i] : x;
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const float y = __shfl_xor(x, o);
        x = y > x ? y : x;
      }
      m[i] = x;
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float x = 0.f;
#pragma unroll
      for (int jt = 0; jt < C / 16; jt++) {
        const float p = sv[jt][i] == neg_inf ? 0.f : __expf(sv[jt][i] - m[i]);
        sv[jt][i] = p;
        x += p;
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) x += __shfl_xor(x, o);
      l[i] = x;
    }
    // exp(s - m_c) into the attention buffer (visible slots) and the
    // probability tile (bf16) for the context product
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = blk * kChunkBlockRows + 4 * lq + i;
      const int64_t g = r / a.Q;
      uint16_t* arow = att + ((b * a.Hq + kvh * a.G + g) * a.Q + t_of[i]) * a.M + s0;
#pragma unroll
      for (int jt = 0; jt < C / 16; jt++) {
        const int jl = jt * 16 + li;
        const uint16_t pb = f32_to_bf16(sv[jt][i]);
        if (row_ok[i] && jl < nact && s0 + jl <= len + t_of[i] && !a.read_only) arow[jl] = pb;
        ptile[(4 * lq + i) * PP + jl] = pb;
      }
      if (li == 0 && r < a.R) {
        if (row_ok[i]) {
          double* cm = a.ws_chunk_ml + ((grp * a.nchunk_max + c) * a.R + r) * 2;
          cm[0] = static_cast<double>(m[i]);
          cm[1] = static_cast<double>(l[i]);
        }
        double* sm = a.ws_seg_ml + (seg * a.R + r) * 2;
        sm[0] = static_cast<double>(m[i]);
        sm[1] = static_cast<double>(l[i]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // context partial o = P V: A = probabilities (row li, slots kk*32 + 8*lq + e)
    uint4 pa[C / 32];
#pragma unroll
    for (int kk = 0; kk < C / 32; kk++) pa[kk] = ld_lds16(ptile + li * PP + kk * 32 + 8 * lq);
#pragma unroll
    for (int nt = 0; nt < DV / 16; nt++) {
      mfma_f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < C / 32; kk++)
        o = mfma_16x16x32(pa[kk], ld_lds16(vt_s + (nt * 16 + li) * VP + kk * 32 + 8 * lq), o);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = blk * kChunkBlockRows + 4 * lq + i;
        if (r < a.R) a.ws_seg_o[(seg * a.R + r) * DV + nt * 16 + li] = o[i];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the next block overwrites the tile
  }
}

}  // namespace kvc

namespace kvc {

// ---- fp32 inputs: the same chunk kernel on the fp64 matrix cores ----------
//
// fp32 scores reach ~1e3 and the probabilities must hold to 1e-5, so the
// products run in fp64 (v_mfma_f64_16x16x4_f64, inputs widened exactly).
// Operand layouts (wave64): lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16], one element each, and receives D[4 i + l / 16][l % 16]
// for i < 4.  K and V stay row-major fp32 in LDS (both operands read one
// element per lane), the probabilities go through a per-wave fp64 tile.
typedef double mfma_f64x4 __attribute__((ext_vector_type(4)));

template <int D, int DV>
__global__ __launch_bounds__(kChunkThreads) void attend_chunk_f32_kernel(StepArgs a) {
  constexpr int C = kChunkSlots;
  constexpr int KP = D + 1;    // row pitches (odd: the 16 lanes of a column
  constexpr int VP = DV + 1;   // read 16 different rows without conflicts)
  constexpr int PP = C + 1;
  static_assert(D % 4 == 0 && DV % 16 == 0, "head sizes");
  __shared__ float k_s[C * KP];
  __shared__ float v_s[C * VP];
  __shared__ double p_s[kChunkWaves][kChunkBlockRows * PP];
  __shared__ RowInfo info_sh;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int RG = chunk_row_groups(a.R);
  const int rg = static_cast<int>(blockIdx.x % RG);
  const int64_t c = (blockIdx.x / RG) % a.nchunk_max;
  const int64_t grp = blockIdx.x / RG / a.nchunk_max;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;

  if (wave == 0) {
    const RowInfo ri = wave_row_info(a.lengths, a.mask, a.Q, a.M, b);
    if (lane == 0) info_sh = ri;
  }
  __syncthreads();
  const RowInfo ri = info_sh;
  if (c == 0 && kvh == 0 && rg == 0 && tid == 0) {
    a.ws_rowinfo[b * 4 + 0] = ri.len;
    a.ws_rowinfo[b * 4 + 1] = ri.n;
    a.ws_rowinfo[b * 4 + 2] = ri.status;
    a.ws_rowinfo[b * 4 + 3] = 0;
  }
  const int64_t len = ri.len, n = ri.n, new_len = len + n;
  const int64_t s0 = c * C;
  const int64_t s1 = s0 + C < a.M ? s0 + C : a.M;

  const int64_t head = b * a.Hk + kvh;
  // slot j of the head at k_head + j * D: the dense cache, or (paged) the
  // chunk's block, which holds all of its slots; null = outside the pool
  const float* k_head = static_cast<const float*>(a.kc_in) + head * a.M * D;
  const float* v_head = static_cast<const float*>(a.vc_in) + head * a.M * DV;
  if (a.paged) {
    const auto* kp = reinterpret_cast<const float*>(slot_row(a, a.kc_in, b, kvh, s0, D * 4));
    const auto* vp = reinterpret_cast<const float*>(slot_row(a, a.vc_in, b, kvh, s0, DV * 4));
    k_head = kp ? kp - s0 * D : nullptr;
    v_head = vp ? vp - s0 * DV : nullptr;
  }
  const float* nk_head = static_cast<const float*>(a.new_key) + head * a.Q * D;
  const float* nv_head = static_cast<const float*>(a.new_value) + head * a.Q * DV;

  // 1. cache writes of the slot range [s0, s1)
  if (rg == 0 && !a.read_only) {  // the chunk's cache writes, once
    // (paged: in place, into the chunk's block, which is the one read)
    uint8_t* kd = a.paged ? const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(k_head))
                          : static_cast<uint8_t*>(a.kc_out) + head * a.M * D * 4;
    uint8_t* vd = a.paged ? const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(v_head))
                          : static_cast<uint8_t*>(a.vc_out) + head * a.M * DV * 4;
    if (kd)
      write_cache_slots(kd, reinterpret_cast<const uint8_t*>(k_head),
                        reinterpret_cast<const uint8_t*>(nk_head), D * 4, s0, s1, len, n,
                        a.out_of_place != 0, tid, kChunkThreads);
    if (vd)
      write_cache_slots(vd, reinterpret_cast<const uint8_t*>(v_head),
                        reinterpret_cast<const uint8_t*>(nv_head), DV * 4, s0, s1, len, n,
                        a.out_of_place != 0, tid, kChunkThreads);
  }
  if (a.R == 0 || c >= row_chunks(len, n, C)) return;
  const int nact = static_cast<int>((s1 < new_len ? s1 : new_len) - s0);

  // 2. K and V rows of the chunk into LDS (slots >= nact as zeros), read in
  // 16-byte pieces, every load issued before the first LDS store
  constexpr int NK = C * (D / 4) / kChunkThreads, NV = C * (DV / 4) / kChunkThreads;
  static_assert(NK * kChunkThreads == C * (D / 4) && NV * kChunkThreads == C * (DV / 4),
                "staging shape");
  float4 kx[NK], vx[NV];
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int idx = tid + i * kChunkThreads, slot = idx / (D / 4), d = (idx % (D / 4)) * 4;
    const int64_t j = s0 + slot;
    kx[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (slot < nact && (j >= len || k_head))
      kx[i] = *reinterpret_cast<const float4*>(j < len ? k_head + j * D + d
                                                       : nk_head + (j - len) * D + d);
  }
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int idx = tid + i * kChunkThreads, slot = idx / (DV / 4), d = (idx % (DV / 4)) * 4;
    const int64_t j = s0 + slot;
    vx[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (slot < nact && (j >= len || v_head))
      vx[i] = *reinterpret_cast<const float4*>(j < len ? v_head + j * DV + d
                                                       : nv_head + (j - len) * DV + d);
  }
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int idx = tid + i * kChunkThreads;
    float* dst = k_s + (idx / (D / 4)) * KP + (idx % (D / 4)) * 4;
    dst[0] = kx[i].x; dst[1] = kx[i].y; dst[2] = kx[i].z; dst[3] = kx[i].w;
  }
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int idx = tid + i * kChunkThreads;
    float* dst = v_s + (idx / (DV / 4)) * VP + (idx % (DV / 4)) * 4;
    dst[0] = vx[i].x; dst[1] = vx[i].y; dst[2] = vx[i].z; dst[3] = vx[i].w;
  }
  __syncthreads();

  // 3. blocks of 16 packed rows, one wave each
  const double scale = a.scale;
  const double neg_inf = -INFINITY;
  const int li = lane % 16, lq = lane / 16;
  const int64_t seg = grp * a.nchunk_max + c;
  const float* qbase = static_cast<const float*>(a.query);
  float* att = static_cast<float*>(a.attention);
  double* ptile = p_s[wave];
  const int nblk = (a.R + kChunkBlockRows - 1) / kChunkBlockRows;
  const int blk_end = (rg + 1) * kChunkWaves < nblk ? (rg + 1) * kChunkWaves : nblk;
  for (int blk = rg * kChunkWaves + wave; blk < blk_end; blk += kChunkWaves) {
    // query row li as A operand: element 4 kk + lq
    double qa[D / 4];
    {
      const int r = blk * kChunkBlockRows + li;
      const int64_t g = r / a.Q, t = r % a.Q;
      const bool ok = r < a.R && t < n;
      const float* qrow = qbase + ((b * a.Hq + kvh * a.G + g) * a.Q + t) * D;
#pragma unroll
      for (int kk = 0; kk < D / 4; kk++) qa[kk] = ok ? static_cast<double>(qrow[4 * kk + lq]) : 0.0;
    }
    // scores: s[jt][i] = S[4 i + lq][16 jt + li]
    mfma_f64x4 s[C / 16];
#pragma unroll
    for (int jt = 0; jt < C / 16; jt++) {
      s[jt] = mfma_f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int kk = 0; kk < D / 4; kk++)
        s[jt] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            qa[kk], static_cast<double>(k_s[(jt * 16 + li) * KP + 4 * kk + lq]), s[jt], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = blk * kChunkBlockRows + 4 * i + lq;
      const int64_t g = r / a.Q, t = r % a.Q;
      const bool row_ok = r < a.R && t < n;
      double sv[C / 16];
      double mx = neg_inf;
#pragma unroll
      for (int jt = 0; jt < C / 16; jt++) {
        const int jl = jt * 16 + li;
        const bool ok = row_ok && jl < nact && s0 + jl <= len + t;
        sv[jt] = ok ? s[jt][i] * scale : neg_inf;
        mx = sv[jt] > mx ? sv[jt] : mx;
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const double y = __shfl_xor(mx, o);
        mx = y > mx ? y : mx;
      }
      double sum = 0.0;
#pragma unroll
      for (int jt = 0; jt < C / 16; jt++) {
        // s - m is exact in fp64; its exponential in fp32 is within ~1e-6
        // relative for every term that is not negligible (s - m > -88)
        sv[jt] = sv[jt] == neg_inf ? 0.0 : static_cast<double>(expf(static_cast<float>(sv[jt] - mx)));
        sum += sv[jt];
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      float* arow = att + ((b * a.Hq + kvh * a.G + g) * a.Q + t) * a.M + s0;
#pragma unroll
      for (int jt = 0; jt < C / 16; jt++) {
        const int jl = jt * 16 + li;
        if (row_ok && jl < nact && s0 + jl <= len + t && !a.read_only)
          arow[jl] = static_cast<float>(sv[jt]);
        ptile[(4 * i + lq) * PP + jl] = sv[jt];
      }
      if (li == 0 && r < a.R) {
        if (row_ok) {
          double* cm = a.ws_chunk_ml + ((grp * a.nchunk_max + c) * a.R + r) * 2;
          cm[0] = mx;
          cm[1] = sum;
        }
        double* sm = a.ws_seg_ml + (seg * a.R + r) * 2;
        sm[0] = mx;
        sm[1] = sum;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // context partial o = P V
#pragma unroll
    for (int nt = 0; nt < DV / 16; nt++) {
      mfma_f64x4 o = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int kk = 0; kk < C / 4; kk++)
        o = __builtin_amdgcn_mfma_f64_16x16x4f64(
            ptile[li * PP + 4 * kk + lq],
            static_cast<double>(v_s[(4 * kk + lq) * VP + nt * 16 + li]), o, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = blk * kChunkBlockRows + 4 * i + lq;
        if (r < a.R) a.ws_seg_o[(seg * a.R + r) * DV + nt * 16 + li] = static_cast<float>(o[i]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the next block overwrites the tile
  }
}

}  // namespace kvc
