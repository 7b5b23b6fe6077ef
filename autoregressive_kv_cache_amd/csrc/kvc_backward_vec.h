// kvc_backward_vec.h -- vector-unit backward of the step for decode-shaped
// heads: bf16 tensors, D = Dv in {64, 128}, at most 8 packed rows per KV
// head (waves of 4 rows for up to 4, of 8 above).  Same gradients as
// kvc_backward.h (see there for the formulas, from "Autoregressive KV-cache
// append and causal attention", the workspace note); what changes is the
// arithmetic's shape.  With so few rows a head's products are
// matrix-vector products: the 16-row fp64 matrix-core tiles of
// kvc_backward.h would be half padding or more, so here every product is a
// per-slot dot product on the vector units, in fp32 (bf16 inputs widen
// exactly; the row statistics are merged in fp64 by bwd_rows_kernel).
//
// Layout of bwd_vstats and bwd_vdq (as attend_stream_kernel, kvc_stream.h):
// for a 64-slot chunk, lane l holds dims [h*64 + (l>>3)*8, +8) of slot
// 8k + (l&7) in piece (k, h), so each 16-byte load covers whole 128-byte
// lines; the 8 partial dot products of a slot are finished by a
// reduce-scatter over lane bits 5, 4 and 3, after which lane l holds slot
// l's value for every packed row.  bwd_vslot computes no dot product and
// gives each lane 8 dims of one slot instead (see there).
//
// Kernels (one wave per (batch row, KV head, run of kBwdVecSlots slots);
// bwd_vslot takes runs of kBwdSlotPassSlots):
//   bwd_vstats: scores s = scale q.K'_j and dP_j = dA_j + dO.V'_j of the
//     run's visible slots, and per packed row the run's max m, sum of
//     e^(s-m) and sum of e^(s-m) dP (the partials bwd_rows_kernel merges);
//     it also stores (s, dP) of every visible slot (fp32, 32 bytes a slot
//     at 4 rows, against 512 bytes of K' and V'), so no later kernel reads V';
//   bwd_vdq: P = e^(s-m)/l and dS = P (dP - sum P dP) from those, and the
//     run's share of dq_r = scale sum_j dS_jr K'_j (summed over the runs by
//     bwd_dq_kernel) -- the one later read of K';
//   bwd_vslot: per slot dK'_j = scale sum_r dS_jr q_r and dV'_j = sum_r
//     P_jr dO_r added to the returned cache's gradient and stored (kept
//     slots to the cache gradient, appended ones to the new rows' gradient,
//     the rest passed through) -- a streaming pass over that gradient.
// Every slot of the cache belongs to one run of bwd_vslot, so the pass-
// through of the returned cache's gradient needs no other kernel.
#pragma once

#include "kvc_backward.h"
#include "kvc_stream.h"

namespace kvc {

typedef unsigned int bwd_u32x4 __attribute__((ext_vector_type(4)));

// 64-slot chunks per wave of the statistics and dq passes.  The run length
// sets how many waves have visible slots against the 2048 the chip runs at
// once, and so whether a last, nearly empty round of waves remains.
// Measured (us per backward call; B=32 decode / one GPU's eighth of the long
// decode / the long decode): 8 chunks 735 / 318 / 1771, 9 chunks
// 725 / 328 / 1650, 10 chunks 738 / 341 / 1662.
constexpr int kBwdVecChunks = 9;
constexpr int kBwdVecSlots = 64 * kBwdVecChunks;    // slots per run (one wave)
constexpr int kBwdVecRows = 8;                      // packed rows a wave holds, at most
// The slot pass in one-chunk runs: it has a wave for every run of the cache
// (pass-through runs included), and more, shorter waves spread its end over
// the chip.  Measured at B = 32, Hk = 8, 8192 slots: the pass took 517 us
// with 512-slot runs, 447 with 256 and 424 with 128, and the whole backward
// call 760 us with 128-slot runs against 730 with 64.  The statistics and
// dq passes, which load every packed row's q and dO per wave, were slower
// with shorter runs (208 -> 232 -> 273 us at 512 -> 256 -> 128) and keep
// longer ones (kBwdVecChunks).
constexpr int kBwdSlotPassChunks = 1;
constexpr int kBwdSlotPassSlots = 64 * kBwdSlotPassChunks;

// Dot products of 8-slot groups k = 0..7 (pieces kb[k * NH + h]) with the
// ROWS row slices qv[r][h], finished so that lane l returns slot l's values.
template <int ROWS, int NH>
__device__ __forceinline__ void lk8_dots(const uint4 (&kb)[8 * NH], const uint4 (&qv)[ROWS][NH],
                                         float (&out)[ROWS]) {
  using Mth = DecodeMath<bf16>;
  const int lane = threadIdx.x % kWave;
  auto partials = [&](int k, float (&p)[ROWS]) {
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      float acc = Mth::dot(qv[r][0], kb[k * NH]);
      if constexpr (NH == 2) {
        acc = Mth::dot2(qv[r][1].x, kb[k * NH + 1].x, acc);
        acc = Mth::dot2(qv[r][1].y, kb[k * NH + 1].y, acc);
        acc = Mth::dot2(qv[r][1].z, kb[k * NH + 1].z, acc);
        acc = Mth::dot2(qv[r][1].w, kb[k * NH + 1].w, acc);
      }
      p[r] = acc;
    }
  };
  float s5[4][ROWS], s4[2][ROWS];
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
  const bool upper = (lane & 8) != 0;
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const float send = upper ? s4[0][r] : s4[1][r], keep = upper ? s4[1][r] : s4[0][r];
    out[r] = keep + dpp<dpp_row_ror(8)>(send);
  }
}

// What the two kernels share for one wave: its head, its run, the rows'
// q and dO slices, the LK8 loads of K' / V' / the returned cache's gradient.
template <int D, int ROWS>
struct BwdVecWave {
  static constexpr int NH = D / 64;
  const BwdArgs& a;
  int lane;
  int64_t grp, b, kvh, j0, len, n, run_slots;
  int Q;
  int r0 = 0;  // the first packed row of the wave's rows (row groups)

  __device__ BwdVecWave(const BwdArgs& args, int64_t wave_id, int64_t nrun,
                        int64_t slots_per_run = kBwdVecSlots)
      : a(args), lane(static_cast<int>(threadIdx.x % kWave)) {
    run_slots = slots_per_run;
    grp = wave_id / nrun;
    j0 = (wave_id % nrun) * slots_per_run;
    b = grp / a.Hk;
    kvh = grp % a.Hk;
    Q = static_cast<int>(a.Q);
  }
  // step query / context row of the wave's row r (packed row r0 + r = g * Q + t)
  __device__ int64_t row_of(int r) const {
    const int rr = r0 + r;
    return (b * a.Hq + kvh * a.G + rr / Q) * a.Q + rr % Q;
  }
  __device__ bool row_valid(int r) const { return r0 + r < a.R && (r0 + r) % Q < n; }
  // slices [h*64 + (lane>>3)*8, +8) of rows r of src ([rows][D]), zeros
  // for rows that are not valid or a null src
  __device__ void load_rows(const void* src, uint4 (&v)[ROWS][NH]) const {
#pragma unroll
    for (int r = 0; r < ROWS; r++)
#pragma unroll
      for (int h = 0; h < NH; h++) {
        const bool ok = src && row_valid(r);
        v[r][h] = ok ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) +
                                                       row_of(r) * D + h * 64 + (lane >> 3) * 8)
                     : make_uint4(0u, 0u, 0u, 0u);
      }
  }
  // LK8 pieces of chunk slots [jb, jb + 64) of K' (cache, or the appended
  // rows for slots in [len, len + n)); zeros past len + n.  Read once per
  // kernel: non-temporal, so they do not displace what is read again --
  // except for row groups (TEMPORAL), whose second wave finds the rows the
  // first one read in L2.
  template <bool TEMPORAL = false>
  __device__ void load_kv(const void* cache, const void* fresh, int64_t jb,
                          uint4 (&v)[8 * NH]) const {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int64_t j = jb + 8 * k + (lane & 7);
      const uint16_t* src = nullptr;
      if (j < len)
        src = static_cast<const uint16_t*>(cache) + (grp * a.M + j) * D;
      else if (j < len + n)
        src = static_cast<const uint16_t*>(fresh) + (grp * a.Q + (j - len)) * D;
#pragma unroll
      for (int h = 0; h < NH; h++) {
        const bwd_u32x4* p = reinterpret_cast<const bwd_u32x4*>(src + h * 64 + (lane >> 3) * 8);
        bwd_u32x4 w{0u, 0u, 0u, 0u};
        if (src) w = TEMPORAL ? *p : __builtin_nontemporal_load(p);
        v[k * NH + h] = make_uint4(w.x, w.y, w.z, w.w);
      }
    }
  }
  // lane l's slot of the chunk at jb and its visibility for packed row r
  __device__ bool visible(int64_t jb, int r) const {
    const int64_t j = jb + lane;
    return row_valid(r) && j <= len + (r0 + r) % Q;
  }
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Scores (natural units, -inf where not visible) and dP of the chunk at jb
// for lane l's slot.
template <int D, int ROWS, bool TEMPORAL>
__device__ __forceinline__ void bwd_vec_chunk(const BwdVecWave<D, ROWS>& W, int64_t jb,
                                              const uint4 (&qv)[ROWS][D / 64],
                                              const uint4 (&dov)[ROWS][D / 64],
                                              uint4 (&kb)[8 * (D / 64)],
                                              float (&s)[ROWS], float (&dp)[ROWS]) {
  constexpr int NH = D / 64;
  const BwdArgs& a = W.a;
  {
    uint4 vb[8 * NH];
    W.template load_kv<TEMPORAL>(a.vc, a.new_value, jb, vb);
    lk8_dots<ROWS, NH>(vb, dov, dp);
  }
  // the V' pieces are dead before the K' ones load (both at once would not
  // fit the registers of two waves per SIMD)
  __builtin_amdgcn_sched_barrier(0);
  W.template load_kv<TEMPORAL>(a.kc, a.new_key, jb, kb);
  lk8_dots<ROWS, NH>(kb, qv, s);
  const int64_t j = jb + W.lane;
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const bool vis = W.visible(jb, r);
    float da = 0.0f;
    if (vis && a.d_att) da = bf16_to_f32(static_cast<const uint16_t*>(a.d_att)[W.row_of(r) * a.M + j]);
    s[r] = vis ? s[r] * a.scale : -INFINITY;
    dp[r] = vis ? dp[r] + da : 0.0f;
  }
}

// A run with no visible slot (all of its slots at or past len + n): the
// gradients of its slots are the returned cache's, passed through (zeros
// for a null one); a plain copy, eight 16-byte pieces in flight per lane.
template <int D, int ROWS>
__device__ void bwd_vec_pass_run(const BwdVecWave<D, ROWS>& W) {
  const BwdArgs& a = W.a;
  const int64_t j1 = W.j0 + W.run_slots < a.M ? W.j0 + W.run_slots : a.M;
  const int64_t pieces = (j1 - W.j0) * D / 8, base = (W.grp * a.M + W.j0) * D;
#pragma unroll
  for (int t = 0; t < 2; t++) {
    const uint4* src = static_cast<const uint4*>(t == 0 ? a.d_kc_out : a.d_vc_out);
    uint4* dst = static_cast<uint4*>(t == 0 ? a.g_kc : a.g_vc);
    src = src ? src + base / 8 : nullptr;
    dst += base / 8;
    for (int64_t p0 = 0; p0 < pieces; p0 += 8 * kWave) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int64_t p = p0 + u * kWave + W.lane;
        v[u] = (src && p < pieces) ? src[p] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int64_t p = p0 + u * kWave + W.lane;
        if (p < pieces) dst[p] = v[u];
      }
    }
  }
}

// The appended rows past n get zero gradients (done by each head's first run).
template <int D, int ROWS>
__device__ void bwd_vec_zero_new_rows(const BwdVecWave<D, ROWS>& W) {
  const BwdArgs& a = W.a;
  for (int64_t i = W.n * D + W.lane * 8; i < a.Q * D; i += kWave * 8) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.g_new_key) + W.grp * a.Q * D + i) =
        make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.g_new_value) + W.grp * a.Q * D + i) =
        make_uint4(0u, 0u, 0u, 0u);
  }
}

// ROWS rows a wave; RG row groups: with RG = 2 two adjacent waves take rows
// [0, ROWS) and [ROWS, 2 ROWS) of the same run, and the second finds the K'
// and V' rows the first loaded in L2 (one wave of 8 rows would need a
// register file of its own per SIMD for the rows' q and dO slices).
template <int D, int ROWS, int RG>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void
bwd_vstats_kernel(BwdArgs a) {
  constexpr int NH = D / 64;
  const int64_t wave_all = blockIdx.x * (kBwdThreads / kWave) + threadIdx.x / kWave;
  const int64_t wave_id = wave_all / RG;
  if (wave_id >= a.B * a.Hk * a.nchunk) return;
  BwdVecWave<D, ROWS> W(a, wave_id, a.nchunk);
  W.r0 = static_cast<int>(wave_all % RG) * ROWS;
  if (W.r0 >= a.R) return;
  bwd_row_info(a, W.b, &W.len, &W.n);
  if (W.n == 0 || W.j0 >= W.len + W.n) return;  // no visible slot: bwd_rows reads nothing here
  uint4 qv[ROWS][NH], dov[ROWS][NH];
  W.load_rows(a.query, qv);
  W.load_rows(a.d_ctx, dov);
  float m[ROWS], l[ROWS], pd[ROWS];  // this lane's running max, sum e^(s-m), sum e^(s-m) dP
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
    pd[r] = 0.0f;
  }
#pragma unroll 1
  for (int c = 0; c < kBwdVecChunks; c++) {
    const int64_t jb = W.j0 + static_cast<int64_t>(c) * 64;
    if (jb >= W.len + W.n) break;
    uint4 kb[8 * NH];
    float s[ROWS], dp[ROWS];
    bwd_vec_chunk<D, ROWS, (RG > 1)>(W, jb, qv, dov, kb, s, dp);
    {  // for the other kernels: (s, dP) of the slot, -inf where not visible
      const int64_t j = jb + W.lane;
#pragma unroll
      for (int r = 0; r < ROWS; r++)
        if (W.r0 + r < a.R && j < W.len + W.n)
          *reinterpret_cast<float2*>(a.ws_sdp + ((W.grp * a.R + W.r0 + r) * a.M + j) * 2) =
              make_float2(s[r], dp[r]);
    }
#pragma unroll
    for (int r = 0; r < ROWS; r++) {
      if (s[r] == -INFINITY) continue;
      const float mn = s[r] > m[r] ? s[r] : m[r];
      const float fo = m[r] == -INFINITY ? 0.0f : expf(m[r] - mn), e = expf(s[r] - mn);
      l[r] = l[r] * fo + e;
      pd[r] = pd[r] * fo + e * dp[r];
      m[r] = mn;
    }
  }
  // merge the lanes in fp64 and store the run's partials
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    if (W.r0 + r >= a.R) continue;
    double md = m[r], ld = l[r], pdd = pd[r];
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const double mo = __shfl_xor(md, o), lo = __shfl_xor(ld, o), po = __shfl_xor(pdd, o);
      const double mn = mo > md ? mo : md;
      if (mn != -INFINITY) {
        const double fa = md == -INFINITY ? 0.0 : exp(md - mn);
        const double fb = mo == -INFINITY ? 0.0 : exp(mo - mn);
        ld = ld * fa + lo * fb;
        pdd = pdd * fa + po * fb;
      }
      md = mn;
    }
    if (W.lane == 0) {
      double* p = a.ws_part + ((W.grp * a.nchunk + wave_id % a.nchunk) * a.R + W.r0 + r) * 4;
      p[0] = md;
      p[1] = ld;
      p[2] = pdd;
      p[3] = 0.0;
    }
  }
}

// P and dS of packed row r at lane l's slot of the chunk at jb, from the
// scores and dP bwd_vstats_kernel stored and the merged row statistics.
template <int D, int ROWS>
__device__ __forceinline__ void bwd_vec_pds(const BwdVecWave<D, ROWS>& W, int64_t jb,
                                            const float (&rm)[ROWS],
                                            const float (&rinv)[ROWS],
                                            const float (&rc)[ROWS],
                                            float (&P)[ROWS], float (&dS)[ROWS]) {
  const BwdArgs& a = W.a;
  const int64_t j = jb + W.lane;
  float2 sd[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; r++)
    sd[r] = (r < a.R && j < W.len + W.n)
                ? *reinterpret_cast<const float2*>(a.ws_sdp + ((W.grp * a.R + r) * a.M + j) * 2)
                : make_float2(-INFINITY, 0.0f);
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    P[r] = sd[r].x == -INFINITY ? 0.0f : expf(sd[r].x - rm[r]) * rinv[r];
    dS[r] = P[r] * (sd[r].y - rc[r]);
  }
}

// The merged statistics of the wave's rows (bwd_rows_kernel): max, 1 / sum
// and sum P dP, one value per wave each (scalar registers).
template <int D, int ROWS>
__device__ __forceinline__ void bwd_vec_row_stats(const BwdVecWave<D, ROWS>& W, float (&rm)[ROWS],
                                                  float (&rinv)[ROWS],
                                                  float (&rc)[ROWS]) {
  const BwdArgs& a = W.a;
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    rm[r] = 0.0f;
    rinv[r] = 0.0f;
    rc[r] = 0.0f;
    if (W.row_valid(r)) {
      const double* st = a.ws_row + W.row_of(r) * 4;
      rm[r] = static_cast<float>(st[0]);
      rinv[r] = st[1] > 0.0 ? static_cast<float>(1.0 / st[1]) : 0.0f;
      rc[r] = static_cast<float>(st[2]);
    }
    rm[r] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(rm[r])));
    rinv[r] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(rinv[r])));
    rc[r] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(rc[r])));
  }
}

// dq: per visible run, dq_r = scale sum_j dS_jr K'_j over the run's slots
// (K' in the LK8 layout: lane l sums its 8 slots of each chunk for its dims,
// then the 8 lanes that hold the same dims add up).
template <int D, int ROWS>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(ROWS <= 4 ? 2 : 1))) void
bwd_vdq_kernel(BwdArgs a) {
  constexpr int NH = D / 64;
  const int64_t wave_id = blockIdx.x * (kBwdThreads / kWave) + threadIdx.x / kWave;
  if (wave_id >= a.B * a.Hk * a.nchunk) return;
  BwdVecWave<D, ROWS> W(a, wave_id, a.nchunk);
  bwd_row_info(a, W.b, &W.len, &W.n);
  if (W.n == 0 || W.j0 >= W.len + W.n) return;  // bwd_dq reads no partial of this run
  const int lane = W.lane;
  float rm[ROWS], rinv[ROWS], rc[ROWS];
  bwd_vec_row_stats<D, ROWS>(W, rm, rinv, rc);
  float dq[ROWS][NH][8];
#pragma unroll
  for (int r = 0; r < ROWS; r++)
#pragma unroll
    for (int h = 0; h < NH; h++)
#pragma unroll
      for (int e = 0; e < 8; e++) dq[r][h][e] = 0.0f;
#pragma unroll 1
  for (int c = 0; c < kBwdVecChunks; c++) {
    const int64_t jb = W.j0 + static_cast<int64_t>(c) * 64;
    if (jb >= W.len + W.n) break;
    uint4 kb[8 * NH];
    W.load_kv(a.kc, a.new_key, jb, kb);
    float P[ROWS], dS[ROWS];
    bwd_vec_pds<D, ROWS>(W, jb, rm, rinv, rc, P, dS);
#pragma unroll
    for (int k = 0; k < 8; k++) {
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        const float ds = __shfl(dS[r], 8 * k + (lane & 7));
#pragma unroll
        for (int h = 0; h < NH; h++) {
          const uint32_t w4[4] = {kb[k * NH + h].x, kb[k * NH + h].y, kb[k * NH + h].z,
                                  kb[k * NH + h].w};
#pragma unroll
          for (int e = 0; e < 4; e++) {
            dq[r][h][2 * e] += ds * bf_lo(w4[e]);
            dq[r][h][2 * e + 1] += ds * bf_hi(w4[e]);
          }
        }
      }
    }
  }
  const int64_t run = wave_id % a.nchunk;
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    if (r >= a.R) continue;
#pragma unroll
    for (int h = 0; h < NH; h++)
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float x = dq[r][h][e];
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        dq[r][h][e] = x;
      }
    if ((lane & 7) == 0) {
      double* p = a.ws_dq + ((W.grp * a.nchunk + run) * a.R + r) * D + (lane >> 3) * 8;
#pragma unroll
      for (int h = 0; h < NH; h++)
#pragma unroll
        for (int e = 0; e < 8; e++) p[h * 64 + e] = static_cast<double>(dq[r][h][e]) * a.scale;
    }
  }
}

// Slot gradients: per run, dK'_j = scale sum_r dS_jr q_r and dV'_j = sum_r
// P_jr dO_r added to the returned cache's gradient and stored (kept slots
// to the cache gradient, appended ones to the new rows' gradient); runs with
// no visible slot are a plain copy.  No K' / V' read: P and dS come from the
// stored scores and dP.  Layout: D / 8 lanes per slot, lane l holding dims
// [(l % (D/8)) * 8, +8) of slot (l / (D/8)) + u * (64 / (D/8)) in step u,
// so each lane keeps only its 8 dims of every row's q and dO.
// Three waves per SIMD: the 4-row form fits them as it is; the 8-row form
// is held to them with 4 loads per batch (a few spilled bytes), which took
// the long decode's backward (131072 slots, 8 rows) from 1827 to 1776 us
// against two waves per SIMD with 8 loads per batch.
template <int D, int ROWS>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(3))) void
bwd_vslot_kernel(BwdArgs a) {
  constexpr int LPS = D / 8, SPI = kWave / LPS, NI = 64 / SPI;  // lanes per slot, slots per step
  constexpr int kSlotBatch = ROWS > 4 ? 4 : 8;  // steps whose loads are issued together
  const int64_t wave_id = blockIdx.x * (kBwdThreads / kWave) + threadIdx.x / kWave;
  const int64_t nrun = (a.M + kBwdSlotPassSlots - 1) / kBwdSlotPassSlots;
  if (wave_id >= a.B * a.Hk * nrun) return;
  BwdVecWave<D, ROWS> W(a, wave_id, nrun, kBwdSlotPassSlots);
  bwd_row_info(a, W.b, &W.len, &W.n);
  const int lane = W.lane;
  if (W.j0 == 0) bwd_vec_zero_new_rows<D, ROWS>(W);
  if (W.n == 0 || W.j0 >= W.len + W.n) {
    bwd_vec_pass_run<D, ROWS>(W);
    return;
  }
  const int col = (lane % LPS) * 8, sl = lane / LPS;
  uint4 qr[ROWS], dor[ROWS];  // this lane's 8 dims of each row's q and dO
#pragma unroll
  for (int r = 0; r < ROWS; r++) {
    const bool ok = W.row_valid(r);
    qr[r] = ok ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.query) +
                                                 W.row_of(r) * D + col)
               : make_uint4(0u, 0u, 0u, 0u);
    dor[r] = ok && a.d_ctx ? *reinterpret_cast<const uint4*>(
                                 static_cast<const uint16_t*>(a.d_ctx) + W.row_of(r) * D + col)
                           : make_uint4(0u, 0u, 0u, 0u);
  }
  float rm[ROWS], rinv[ROWS], rc[ROWS];
  bwd_vec_row_stats<D, ROWS>(W, rm, rinv, rc);
#pragma unroll 1
  for (int c = 0; c < kBwdSlotPassChunks; c++) {
    const int64_t jb = W.j0 + static_cast<int64_t>(c) * 64;
    if (jb >= a.M) break;
    float P[ROWS], dS[ROWS];
    bwd_vec_pds<D, ROWS>(W, jb, rm, rinv, rc, P, dS);
#pragma unroll
    for (int t = 0; t < 2; t++) {  // t = 0: keys, t = 1: values
      const uint16_t* pass = static_cast<const uint16_t*>(t == 0 ? a.d_kc_out : a.d_vc_out);
      uint16_t* gcache = static_cast<uint16_t*>(t == 0 ? a.g_kc : a.g_vc);
      uint16_t* gnew = static_cast<uint16_t*>(t == 0 ? a.g_new_key : a.g_new_value);
      float wsrc[ROWS];
      uint4 src[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; r++) {
        wsrc[r] = t == 0 ? dS[r] * a.scale : P[r];
        src[r] = t == 0 ? qr[r] : dor[r];
      }
#pragma unroll 1
      for (int ub = 0; ub < NI; ub += kSlotBatch) {
        uint4 x[kSlotBatch];  // pass-through pieces, all in flight together
#pragma unroll
        for (int u = 0; u < kSlotBatch; u++) {
          const int64_t j = jb + (ub + u) * SPI + sl;
          x[u] = (pass && j < a.M)
                     ? *reinterpret_cast<const uint4*>(pass + (W.grp * a.M + j) * D + col)
                     : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kSlotBatch; u++) {
          const int64_t j = jb + (ub + u) * SPI + sl;
          float wk[ROWS];
#pragma unroll
          for (int r = 0; r < ROWS; r++) wk[r] = __shfl(wsrc[r], (ub + u) * SPI + sl);
          if (j >= a.M) continue;
          const uint32_t xw[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            v[2 * e] = bf_lo(xw[e]);
            v[2 * e + 1] = bf_hi(xw[e]);
          }
#pragma unroll
          for (int r = 0; r < ROWS; r++) {
            const uint32_t sw[4] = {src[r].x, src[r].y, src[r].z, src[r].w};
#pragma unroll
            for (int e = 0; e < 4; e++) {
              v[2 * e] += wk[r] * bf_lo(sw[e]);
              v[2 * e + 1] += wk[r] * bf_hi(sw[e]);
            }
          }
          uint32_t y[4];
#pragma unroll
          for (int e = 0; e < 4; e++)
            y[e] = static_cast<uint32_t>(f32_to_bf16(v[2 * e])) |
                   (static_cast<uint32_t>(f32_to_bf16(v[2 * e + 1])) << 16);
          const uint4 out{y[0], y[1], y[2], y[3]};
          uint4* at = reinterpret_cast<uint4*>(gcache + (W.grp * a.M + j) * D + col);
          if (j >= W.len && j < W.len + W.n) {  // appended: its gradient goes to the new row
            *reinterpret_cast<uint4*>(gnew + (W.grp * a.Q + (j - W.len)) * D + col) = out;
            *at = make_uint4(0u, 0u, 0u, 0u);
          } else {
            *at = out;
          }
        }
      }
    }
  }
}

}  // namespace kvc
