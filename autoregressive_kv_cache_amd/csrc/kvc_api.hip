// kvc_api.hip -- host side of the C ABI declared in include/kvc.h: argument
// checks, kernel plan, workspace layout and launches on the caller's stream.
// No allocation, no synchronisation, no state kept between calls.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/kvc.h"
#include "kvc_combine.h"
#include "kvc_common.h"
#include "kvc_generic.h"

namespace {

using kvc::StepArgs;

constexpr int64_t kMaxElems = int64_t(1) << 46;    // per tensor
constexpr int64_t kMaxWorkgroups = int64_t(1) << 24;

// a * b with an overflow / limit check
bool mul_ok(int64_t a, int64_t b, int64_t limit, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > limit / a) return false;
  *out = a * b;
  return *out <= limit;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Plan {
  kvc_plan pub;
  size_t off_rowinfo, off_ml, off_o;
};

int check_dims(const kvc_dims* d, int dtype) {
  if (!d) return KVC_ERR_NULL;
  if (d->B < 1 || d->Hq < 1 || d->Hk < 1 || d->M < 1 || d->D < 1 || d->Dv < 1 || d->Q < 0)
    return KVC_ERR_SHAPE;
  if (d->Hq % d->Hk != 0) return KVC_ERR_SHAPE;
  if (dtype != KVC_F32 && dtype != KVC_BF16) return KVC_ERR_DTYPE;
  int64_t x, y;
  // every tensor's element count must stay addressable with 64-bit offsets
  if (!mul_ok(d->B, d->Hk, kMaxElems, &x) || !mul_ok(x, d->M, kMaxElems, &y) ||
      !mul_ok(y, d->D > d->Dv ? d->D : d->Dv, kMaxElems, &y))
    return KVC_ERR_SHAPE;
  if (!mul_ok(d->B, d->Hq, kMaxElems, &x) || !mul_ok(x, d->Q, kMaxElems, &x) ||
      !mul_ok(x, d->M > d->D ? (d->M > d->Dv ? d->M : d->Dv) : (d->D > d->Dv ? d->D : d->Dv),
              kMaxElems, &y))
    return KVC_ERR_SHAPE;
  if (d->Hq / d->Hk > (int64_t(1) << 20) || d->Q > (int64_t(1) << 20)) return KVC_ERR_SHAPE;
  if ((d->Hq / d->Hk) * d->Q > (int64_t(1) << 20)) return KVC_ERR_SHAPE;
  return KVC_OK;
}

int make_plan(const kvc_dims* d, int dtype, Plan* p) {
  int rc = check_dims(d, dtype);
  if (rc != KVC_OK) return rc;
  std::memset(p, 0, sizeof *p);
  const int64_t R = (d->Hq / d->Hk) * d->Q;
  p->pub.rows = static_cast<int32_t>(R);
  p->pub.path = 0;
  p->pub.rows_per_tile = kvc::kGenericRowsPerTile;
  p->pub.split = kvc::kGenericSplit;
  p->pub.row_tiles = static_cast<int32_t>(R == 0 ? 1 : (R + p->pub.rows_per_tile - 1) / p->pub.rows_per_tile);
  p->pub.nsplit = (d->M + p->pub.split - 1) / p->pub.split;

  int64_t groups, wgs, parts, obytes;
  if (!mul_ok(d->B, d->Hk, kMaxElems, &groups) ||
      !mul_ok(groups, p->pub.row_tiles, kMaxElems, &wgs) ||
      !mul_ok(wgs, p->pub.nsplit, kMaxWorkgroups, &wgs))
    return KVC_ERR_SHAPE;
  if (!mul_ok(groups, p->pub.nsplit, kMaxElems, &parts) || !mul_ok(parts, R, kMaxElems, &parts) ||
      !mul_ok(parts, d->Dv, kMaxElems, &obytes))
    return KVC_ERR_SHAPE;
  size_t off = 0;
  p->off_rowinfo = off;
  off = align_up(off + static_cast<size_t>(d->B) * 4 * sizeof(int64_t), 256);
  p->off_ml = off;
  off = align_up(off + static_cast<size_t>(parts) * 2 * sizeof(double), 256);
  p->off_o = off;
  off = align_up(off + static_cast<size_t>(obytes) * sizeof(float), 256);
  p->pub.workspace_bytes = off;
  return KVC_OK;
}

int check_scale(int has_scale, double scale, int64_t D, double* out) {
  if (!has_scale) {
    *out = 1.0 / std::sqrt(static_cast<double>(D));
    return KVC_OK;
  }
  if (!std::isfinite(scale) || !(scale > 0.0)) return KVC_ERR_SCALE;
  *out = scale;
  return KVC_OK;
}

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

template <typename T>
void launch_all(const Plan& p, StepArgs& a, hipStream_t stream, const kvc_events* ev) {
  const int64_t groups = a.B * a.Hk;
  const dim3 grid_attend(static_cast<unsigned>(groups * a.row_tiles * a.nsplit));
  const dim3 grid_combine(static_cast<unsigned>(groups * a.nsplit));
  if (ev && ev->start) hipEventRecord(static_cast<hipEvent_t>(ev->start), stream);
  hipLaunchKernelGGL(kvc::attend_generic_kernel<T>, grid_attend, dim3(kvc::kGenericThreads), 0,
                     stream, a);
  if (ev && ev->stop) hipEventRecord(static_cast<hipEvent_t>(ev->stop), stream);
  hipLaunchKernelGGL(kvc::combine_kernel<T>, grid_combine, dim3(kvc::kCombineThreads), 0, stream,
                     a);
  (void)p;
}

int run_step(const kvc_dims* d, int dtype, int has_scale, double scale, const void* query,
             const void* new_key, const void* new_value, const void* kc_in, const void* vc_in,
             void* kc_out, void* vc_out, bool out_of_place, const int64_t* lengths,
             const uint8_t* mask, int64_t* lengths_out, void* attention, void* context,
             int32_t* row_status, void* workspace, size_t workspace_bytes, void* stream,
             const kvc_events* events) {
  Plan p;
  int rc = make_plan(d, dtype, &p);
  if (rc != KVC_OK) return rc;
  double sc;
  rc = check_scale(has_scale, scale, d->D, &sc);
  if (rc != KVC_OK) return rc;

  if (!kc_in || !vc_in || !kc_out || !vc_out || !lengths || !lengths_out) return KVC_ERR_NULL;
  if (d->Q > 0 && (!query || !new_key || !new_value || !mask || !attention || !context))
    return KVC_ERR_NULL;
  if (p.pub.workspace_bytes > 0 && !workspace) return KVC_ERR_NULL;
  if (workspace_bytes < p.pub.workspace_bytes) return KVC_ERR_WORKSPACE;

  const size_t e = dtype == KVC_F32 ? 4 : 2;
  const size_t B = d->B, Hq = d->Hq, Hk = d->Hk, Q = d->Q, M = d->M, D = d->D, Dv = d->Dv;
  const Range r_q{query, B * Hq * Q * D * e}, r_nk{new_key, B * Hk * Q * D * e},
      r_nv{new_value, B * Hk * Q * Dv * e}, r_kin{kc_in, B * Hk * M * D * e},
      r_vin{vc_in, B * Hk * M * Dv * e}, r_len{lengths, B * 8}, r_mask{mask, B * Q},
      r_kout{kc_out, B * Hk * M * D * e}, r_vout{vc_out, B * Hk * M * Dv * e},
      r_lout{lengths_out, B * 8}, r_att{attention, B * Hq * Q * M * e},
      r_ctx{context, B * Hq * Q * Dv * e}, r_st{row_status, row_status ? B * 4 : 0},
      r_ws{workspace, p.pub.workspace_bytes};
  const bool len_in_place = !out_of_place && lengths_out == lengths;
  const Range inputs[] = {r_q, r_nk, r_nv, r_mask, len_in_place ? Range{nullptr, 0} : r_len};
  const Range caches_in[] = {r_kin, r_vin};
  const Range outs[] = {r_kout, r_vout, len_in_place ? Range{nullptr, 0} : r_lout,
                        r_att, r_ctx, r_st, r_ws};
  const int n_out = out_of_place ? 7 : 5;
  const Range* outp = out_of_place ? outs : outs + 2;
  for (int i = 0; i < n_out; i++) {
    for (const Range& in : inputs)
      if (overlap(outp[i], in)) return KVC_ERR_ALIAS;
    for (const Range& c : caches_in)
      if (overlap(outp[i], c)) return KVC_ERR_ALIAS;
    for (int j = i + 1; j < n_out; j++)
      if (overlap(outp[i], outp[j])) return KVC_ERR_ALIAS;
  }
  if (len_in_place) {  // lengths itself must still not overlap other buffers
    const Range others[] = {r_q, r_nk, r_nv, r_mask, r_kin, r_vin, r_att, r_ctx, r_st, r_ws};
    for (const Range& o : others)
      if (overlap(r_len, o)) return KVC_ERR_ALIAS;
  }
  if (!out_of_place) {  // the two caches are written in place
    for (const Range& in : inputs)
      for (const Range& c : caches_in)
        if (overlap(in, c)) return KVC_ERR_ALIAS;
    if (overlap(r_kin, r_vin)) return KVC_ERR_ALIAS;
  }

  StepArgs a;
  std::memset(&a, 0, sizeof a);
  a.B = d->B; a.Hq = d->Hq; a.Hk = d->Hk; a.Q = d->Q; a.M = d->M; a.D = d->D; a.Dv = d->Dv;
  a.G = static_cast<int32_t>(d->Hq / d->Hk);
  a.R = p.pub.rows;
  a.rows_per_tile = p.pub.rows_per_tile;
  a.row_tiles = p.pub.row_tiles;
  a.S = p.pub.split;
  a.nsplit = p.pub.nsplit;
  a.scale = sc;
  a.out_of_place = out_of_place ? 1 : 0;
  a.query = query; a.new_key = new_key; a.new_value = new_value;
  a.kc_in = kc_in; a.vc_in = vc_in; a.kc_out = kc_out; a.vc_out = vc_out;
  a.lengths = lengths; a.mask = mask; a.attention = attention; a.context = context;
  a.lengths_out = lengths_out; a.row_status = row_status;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.ws_rowinfo = reinterpret_cast<int64_t*>(ws + p.off_rowinfo);
  a.ws_ml = reinterpret_cast<double*>(ws + p.off_ml);
  a.ws_o = reinterpret_cast<float*>(ws + p.off_o);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == KVC_F32)
    launch_all<float>(p, a, s, events);
  else
    launch_all<kvc::bf16>(p, a, s, events);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

}  // namespace

extern "C" {

size_t kvc_workspace_bytes(const kvc_dims* dims, int dtype) {
  Plan p;
  return make_plan(dims, dtype, &p) == KVC_OK ? p.pub.workspace_bytes : 0;
}

int kvc_plan_step(const kvc_dims* dims, int dtype, kvc_plan* plan) {
  if (!plan) return KVC_ERR_NULL;
  Plan p;
  const int rc = make_plan(dims, dtype, &p);
  if (rc == KVC_OK) *plan = p.pub;
  return rc;
}

int kvc_step_out_of_place(const kvc_dims* dims, int dtype, int has_scale, double scale,
                          const void* query, const void* new_key, const void* new_value,
                          const void* key_cache, const void* value_cache, const int64_t* lengths,
                          const uint8_t* append_mask, void* key_cache_out, void* value_cache_out,
                          int64_t* lengths_out, void* attention, void* context,
                          int32_t* row_status, void* workspace, size_t workspace_bytes,
                          void* stream, const kvc_events* events) {
  return run_step(dims, dtype, has_scale, scale, query, new_key, new_value, key_cache,
                  value_cache, key_cache_out, value_cache_out, true, lengths, append_mask,
                  lengths_out, attention, context, row_status, workspace, workspace_bytes, stream,
                  events);
}

int kvc_step_inplace(const kvc_dims* dims, int dtype, int has_scale, double scale,
                     const void* query, const void* new_key, const void* new_value,
                     void* key_cache, void* value_cache, const int64_t* lengths,
                     const uint8_t* append_mask, int64_t* lengths_out, void* attention,
                     void* context, int32_t* row_status, void* workspace, size_t workspace_bytes,
                     void* stream, const kvc_events* events) {
  return run_step(dims, dtype, has_scale, scale, query, new_key, new_value, key_cache,
                  value_cache, key_cache, value_cache, false, lengths, append_mask, lengths_out,
                  attention, context, row_status, workspace, workspace_bytes, stream, events);
}

const char* kvc_status_string(int code) {
  switch (code) {
    case KVC_OK: return "ok";
    case KVC_ERR_NULL: return "a required pointer is NULL";
    case KVC_ERR_SHAPE: return "sizes out of range, Hq not a multiple of Hk, or too large";
    case KVC_ERR_DTYPE: return "unsupported dtype";
    case KVC_ERR_SCALE: return "scale must be finite and > 0";
    case KVC_ERR_WORKSPACE: return "workspace too small";
    case KVC_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case KVC_ERR_HIP: return "a HIP launch failed";
    case KVC_ROW_BAD_LENGTH: return "row rejected: length outside [0, M]";
    case KVC_ROW_OVERFLOW: return "row rejected: length + n exceeds M";
    case KVC_ROW_NOT_PREFIX: return "row rejected: append mask is not a prefix";
    default: return "unknown code";
  }
}

}  // extern "C"
