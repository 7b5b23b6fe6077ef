// kvc_combine_stream.h -- the combine kernel of the bf16 stream path: turns
// what attend_stream_kernel (kvc_stream.h) left in the workspace into the
// step's outputs.
//
// For a valid packed query row with segments (m_s, l_s, o_s) (m in log2
// units, l_s = sum_j exp2(s_j - m_s), o_s = sum_j exp2(s_j - m_s) v_j):
//   m = max m_s,  l = sum l_s exp2(m_s - m),  context = sum o_s exp2(m_s - m) / l,
// and slot j of chunk x, stored as exp2(s_j - m_ref(x)), becomes
// exp2(s_j - m) / l after one multiplication by exp2(m_ref(x) - m) / l --
// the normalised softmax of "Autoregressive KV-cache append and causal
// attention" (Required behavior).  Slots after length + t and whole invalid
// rows get exact zeros.  A re-attention's sink (a logit in natural units)
// joins the merge as one more term with no value row.
//
// Grid, roles and the cache work (the in-place append of the step's rows,
// the out-of-place tail copy) are those of combine_kernel (kvc_combine.h):
// one workgroup per (group, range of CS slots), plus one per group that
// merges the contexts; wave w of a workgroup owns packed row w of its block.
#pragma once

#include "kvc_combine.h"
#include "kvc_stream.h"

namespace kvc {

__global__ __launch_bounds__(kCombineThreads) void combine_stream_kernel(StepArgs a) {
  constexpr int VPL = kCombineVecPerLane;
  constexpr int C = kStreamChunk;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int64_t ncw = ceil_div(a.M, a.CS);
  const int64_t nrb = a.R > 0 ? ceil_div(a.R, kCombineWaves) : 1;
  // read-only (re-attention): the context role of each group alone (see
  // combine_kernel); the attend kernel kept no exp values either
  const int64_t rb = blockIdx.x % nrb;
  const int64_t k = a.read_only ? ncw : (blockIdx.x / nrb) % (ncw + 1);
  const int64_t grp = a.read_only ? blockIdx.x / nrb : blockIdx.x / nrb / (ncw + 1);
  const bool ctx_role = k == ncw;
  const int64_t b = grp / a.Hk, kvh = grp % a.Hk;
  // the row record and the stream header in one round of loads
  const int64_t len = a.ws_rowinfo[b * 4 + 0];
  const int64_t n = a.ws_rowinfo[b * 4 + 1];
  const int32_t status = static_cast<int32_t>(a.ws_rowinfo[b * 4 + 2]);
  const int64_t first_chunk = a.ws_rowinfo[b * 4 + 3];
  const int64_t hdr_nc = a.ws_hdr[0], hdr_pe = a.ws_hdr[1];
  const int64_t nc = stream_chunks(len, n, C);
  const int64_t len_chunks = (len + C - 1) / C;  // cached chunks; the appended rows follow
  const int64_t xg = first_chunk + kvh * nc;     // the group's first flattened chunk

  if ((a.read_only ? ctx_role : k == 0) && kvh == 0 && rb == 0 && tid == 0) {
    a.lengths_out[b] = len + n;
    if (a.row_status) a.row_status[b] = status;
  }
  const int64_t e0 = ctx_role ? a.M : k * a.CS;
  const int64_t e1 = e0 + a.CS < a.M ? e0 + a.CS : a.M;

  if (ctx_role && rb == 0 && !a.out_of_place && !a.read_only && n > 0) {
    // in place: the appended rows go to their cache slots (the attend
    // kernel read them from new_key / new_value)
    const int64_t kb = a.D * 2, vb = a.Dv * 2;
    const uint8_t* nk = static_cast<const uint8_t*>(a.new_key) + grp * a.Q * kb;
    const uint8_t* nv = static_cast<const uint8_t*>(a.new_value) + grp * a.Q * vb;
    if (!a.paged) {
      copy_bytes(static_cast<uint8_t*>(a.kc_out) + (grp * a.M + len) * kb, nk, n * kb, tid,
                 kCombineThreads);
      copy_bytes(static_cast<uint8_t*>(a.vc_out) + (grp * a.M + len) * vb, nv, n * vb, tid,
                 kCombineThreads);
    } else {
      // one row at a time: consecutive slots may lie in different blocks
      for (int64_t t = 0; t < n; t++) {
        uint8_t* kd = const_cast<uint8_t*>(slot_row(a, a.kc_out, b, kvh, len + t, kb));
        uint8_t* vd = const_cast<uint8_t*>(slot_row(a, a.vc_out, b, kvh, len + t, vb));
        if (kd) copy_bytes(kd, nk + t * kb, kb, tid, kCombineThreads);
        if (vd) copy_bytes(vd, nv + t * vb, vb, tid, kCombineThreads);
      }
    }
  }
  if (rb == 0 && a.out_of_place && a.combine_copies_tail) {
    const int64_t cover = n > 0 ? len + n : 0;
    const int64_t j0 = e0 > cover ? e0 : cover;
    if (j0 < e1) {
      const int64_t kb = a.D * 2, vb = a.Dv * 2;
      const int64_t hk = grp * a.M;
      copy_bytes(static_cast<uint8_t*>(a.kc_out) + (hk + j0) * kb,
                 static_cast<const uint8_t*>(a.kc_in) + (hk + j0) * kb, (e1 - j0) * kb, tid,
                 kCombineThreads);
      copy_bytes(static_cast<uint8_t*>(a.vc_out) + (hk + j0) * vb,
                 static_cast<const uint8_t*>(a.vc_in) + (hk + j0) * vb, (e1 - j0) * vb, tid,
                 kCombineThreads);
    }
  }

  const int64_t r = rb * kCombineWaves + wave;
  if (r >= a.R) return;
  const int64_t R = a.R;
  const int64_t g = r / a.Q, t = r % a.Q;
  const int64_t row = (b * a.Hq + kvh * a.G + g) * a.Q + t;
  const int64_t lim = t < n ? len + t + 1 : 0;  // visible slots [0, lim)
  uint16_t* arow = static_cast<uint16_t*>(a.attention) + row * a.M;
  uint16_t* ctx = static_cast<uint16_t*>(a.context) + row * a.Dv;
  const SegRange sr = group_segments(a, grp, kvh, nc, first_chunk, hdr_nc, hdr_pe);
  const bool vec = (reinterpret_cast<uintptr_t>(a.attention) % 16 == 0) && (a.M % 8 == 0);

  // chunk of slot j (< lim) and its position in that chunk
  auto chunk_of = [&](int64_t j) { return j < len ? j / C : len_chunks; };
  auto pos_of = [&](int64_t j) { return j < len ? j % C : j - len; };
  auto exp_at = [&](int64_t j) {
    return bf16_to_f32(a.ws_pexp[((xg + chunk_of(j)) * R + r) * C + pos_of(j)]);
  };
  auto ref_at = [&](int64_t j) { return a.ws_cref[(xg + chunk_of(j)) * R + r]; };

  // ---- first pass of the range: its loads go out before the statistics ----
  // a vector of 8 slots inside one cached chunk is one 16-byte load; the few
  // that reach the appended rows (their chunk starts at slot len) go element
  // by element after the statistics
  const int64_t nvec = (e1 - e0) / 8;
  uint4 x[VPL];
  float ref[VPL];
  auto load_vec = [&](int v, int64_t vi) {
    const int64_t base = e0 + vi * 8;
    const bool whole = vi < nvec && base + 8 <= lim && base + 8 <= len;
    x[v] = make_uint4(0, 0, 0, 0);
    ref[v] = 0.0f;
    if (whole) {
      const int64_t ch = xg + base / C;
      const nt_u32x4 w = __builtin_nontemporal_load(
          reinterpret_cast<const nt_u32x4*>(a.ws_pexp + (ch * R + r) * C + base % C));
      x[v] = make_uint4(w.x, w.y, w.z, w.w);
      ref[v] = a.ws_cref[ch * R + r];
    }
  };
  if (vec) {
#pragma unroll
    for (int v = 0; v < VPL; v++) load_vec(v, v * kWave + lane);
  }

  // segment statistics of the first kWave segments (lane s holds segment s)
  // and, for the context role, the first batch of segment partials
  constexpr int SB = 16;
  const bool do_ctx = ctx_role && t < n && sr.count > 0;
  float seg_m0 = -INFINITY, seg_l0 = 0;
  if (t < n && lane < sr.count) {
    const float* ml = a.ws_seg2 + ((sr.first + lane) * R + r) * 2;
    seg_m0 = ml[0];
    seg_l0 = ml[1];
  }
  float cv[SB][2];
  auto load_batch = [&](int64_t s1, int64_t dv0) {
#pragma unroll
    for (int s = 0; s < SB; s++) {
      const float* op = a.ws_seg_o + ((sr.first + s1 + s) * R + r) * a.Dv;
#pragma unroll
      for (int q = 0; q < 2; q++) {
        const int64_t dv = dv0 + q * kWave + lane;
        cv[s][q] = (s1 + s < sr.count && dv < a.Dv) ? op[dv] : 0.0f;
      }
    }
  };
  if (do_ctx) load_batch(0, 0);

  // ---- m and 1/l of the row over its segments (log2 units) ----
  float m = -INFINITY, l = 0;
  if (t < n) {
    auto merge = [&](float ms, float ls) {
      if (ls > 0.0f) {
        const float mn = ms > m ? ms : m;
        l = (m == -INFINITY ? 0.0f : l * exp2_fast(m - mn)) + ls * exp2_fast(ms - mn);
        m = mn;
      }
    };
    merge(seg_m0, seg_l0);
    for (int64_t s = kWave + lane; s < sr.count; s += kWave) {
      const float* ml = a.ws_seg2 + ((sr.first + s) * R + r) * 2;
      merge(ml[0], ml[1]);
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const float mo = __shfl_xor(m, o), lo = __shfl_xor(l, o);
      const float mn = mo > m ? mo : m;
      if (mn != -INFINITY)
        l = (m == -INFINITY ? 0.0f : l * exp2_fast(m - mn)) +
            (mo == -INFINITY ? 0.0f : lo * exp2_fast(mo - mn));
      m = mn;
    }
    if (a.sinks) {  // the head's sink: one more logit, no value row
      const float sk = a.sinks[kvh * a.G + g] * kLog2e;
      const float mn = sk > m ? sk : m;
      l = (m == -INFINITY ? 0.0f : l * exp2_fast(m - mn)) + exp2_fast(sk - mn);
      m = mn;
    }
  }
  const float inv_l = l > 0 ? 1.0f / l : 0.0f;
  auto factor = [&](float mr) { return exp2_fast(mr - m) * inv_l; };

  // ---- rescale the visible slots, zero the rest ----
  if (vec) {
    for (int64_t v0 = 0; v0 < nvec; v0 += VPL * kWave) {
      if (v0 > 0) {
#pragma unroll
        for (int v = 0; v < VPL; v++) load_vec(v, v0 + v * kWave + lane);
      }
#pragma unroll
      for (int v = 0; v < VPL; v++) {
        const int64_t vi = v0 + v * kWave + lane;
        const int64_t base = e0 + vi * 8;
        if (vi < nvec) {
          uint32_t o[4];
          if (base + 8 <= lim && base + 8 <= len) {
            const float f = factor(ref[v]);
            const uint32_t* w = reinterpret_cast<const uint32_t*>(&x[v]);
#pragma unroll
            for (int e = 0; e < 4; e++) {
              const uint32_t lo = bf16_bits(__uint_as_float(w[e] << 16) * f);
              const uint32_t hi = bf16_bits(__uint_as_float(w[e] & 0xffff0000u) * f);
              o[e] = lo | (hi << 16);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; e++) {
              uint32_t pair = 0;
#pragma unroll
              for (int h = 0; h < 2; h++) {
                const int64_t j = base + 2 * e + h;
                const uint32_t bits = j < lim ? bf16_bits(exp_at(j) * factor(ref_at(j))) : 0u;
                pair |= bits << (16 * h);
              }
              o[e] = pair;
            }
          }
          const nt_u32x4 wv = {o[0], o[1], o[2], o[3]};
          __builtin_nontemporal_store(wv, reinterpret_cast<nt_u32x4*>(arow + base));
        }
      }
    }
  } else {
    for (int64_t j = e0 + lane; j < e1; j += kWave)
      arow[j] = j < lim ? bf16_bits(exp_at(j) * factor(ref_at(j))) : uint16_t(0);
  }

  // ---- context of the rows this range owns ----
  if (!ctx_role) return;
  if (!do_ctx) {
    for (int64_t dv = lane; dv < a.Dv; dv += kWave) ctx[dv] = 0;
    return;
  }
  // lanes own dims dv0 + q * 64 + lane, q < 2
  for (int64_t dv0 = 0; dv0 < a.Dv; dv0 += 2 * kWave) {
    float o[2] = {0, 0};
    for (int64_t s0 = 0; s0 < sr.count; s0 += kWave) {
      // weight of segment s0 + lane; broadcast one segment at a time
      float w = 0;
      if (s0 == 0) {
        w = seg_l0 > 0.0f ? factor(seg_m0) : 0.0f;
      } else if (s0 + lane < sr.count) {
        const float* ml = a.ws_seg2 + ((sr.first + s0 + lane) * R + r) * 2;
        w = ml[1] > 0.0f ? factor(ml[0]) : 0.0f;
      }
      const int64_t nsg = sr.count - s0 < kWave ? sr.count - s0 : kWave;
      for (int64_t s1 = 0; s1 < nsg; s1 += SB) {
        if (dv0 > 0 || s0 > 0 || s1 > 0) load_batch(s0 + s1, dv0);
#pragma unroll
        for (int s = 0; s < SB; s++) {
          const float ws = __shfl(w, static_cast<int>(s1 + s));  // 0 past the last segment
#pragma unroll
          for (int q = 0; q < 2; q++) o[q] += ws * cv[s][q];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int64_t dv = dv0 + q * kWave + lane;
      if (dv < a.Dv) ctx[dv] = bf16_bits(o[q]);
    }
  }
}

}  // namespace kvc
