// kvc_backward_api.hip -- host side of the backward entry points of
// include/kvc.h (kvc_backward_workspace_bytes, kvc_step_backward): checks,
// workspace layout and the four launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/kvc.h"
#include "kvc_backward.h"
#include "kvc_backward_generic.h"
#include "kvc_backward_vec.h"
#include "kvc_host.h"

namespace {

using namespace kvc_host;

constexpr int64_t kMaxBwdWorkgroups = int64_t(1) << 30;

// Backward: fp32 or bf16 tensors, head sizes with a chunk kernel below.
struct BwdEntry {
  int dtype;
  int64_t D, Dv;
  void (*stats)(const kvc::BwdArgs&, hipStream_t);
  void (*chunk)(const kvc::BwdArgs&, hipStream_t);
  void (*dq)(const kvc::BwdArgs&, hipStream_t);
};
template <typename T, int D, int DV>
void launch_bwd_stats(const kvc::BwdArgs& a, hipStream_t s) {
  static_assert(kvc::kBwdThreads % D == 0, "bwd_dq spreads a row's D columns over the workgroup");
  hipLaunchKernelGGL((kvc::bwd_stats_kernel<T, D, DV>),
                     dim3(static_cast<unsigned>(a.B * a.Hk * a.nchunk * a.row_groups)),
                     dim3(kvc::kBwdThreads), 0, s, a);
}
template <typename T, int D, int DV>
void launch_bwd_chunk(const kvc::BwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B * a.Hk * a.nchunk));
  if (a.R > kvc::kBwdRowTile)
    hipLaunchKernelGGL((kvc::bwd_chunk_kernel<T, D, DV, kvc::kBwdChunkRowsWide>), grid,
                       dim3(kvc::kBwdThreads), 0, s, a);
  else
    hipLaunchKernelGGL((kvc::bwd_chunk_kernel<T, D, DV, kvc::kBwdRowTile>), grid,
                       dim3(kvc::kBwdThreads), 0, s, a);
}
template <typename T>
void launch_bwd_dq(const kvc::BwdArgs& a, hipStream_t s) {
  const int64_t rows = a.B * a.Hq * a.Q;
  hipLaunchKernelGGL((kvc::bwd_dq_kernel<T>), dim3(static_cast<unsigned>(rows)),
                     dim3(kvc::kBwdThreads), 0, s, a);
}
#define KVC_BWD(T, CODE, D, DV)                                                            \
  {CODE, D, DV, &launch_bwd_stats<T, D, DV>, &launch_bwd_chunk<T, D, DV>, &launch_bwd_dq<T>}
const BwdEntry kBwdTable[] = {
    KVC_BWD(float, KVC_F32, 64, 64),       KVC_BWD(float, KVC_F32, 128, 128),
    KVC_BWD(float, KVC_F32, 64, 32),       KVC_BWD(kvc::bf16, KVC_BF16, 64, 64),
    KVC_BWD(kvc::bf16, KVC_BF16, 128, 128), KVC_BWD(kvc::bf16, KVC_BF16, 64, 32),
};
#undef KVC_BWD
// The vector-unit kernels of kvc_backward_vec.h: bf16, D = Dv in {64, 128},
// at most kBwdVecRows packed rows per KV head (waves of 4 rows up to 4, of 8
// above).
// which: 0 statistics, 1 dq, 2 slot gradients
// (the slot pass runs over kBwdSlotPassSlots-slot runs: at most the 64-slot
// chunk count the host checks bound for every grid)
template <int D, int ROWS>
void launch_bwd_vec(const kvc::BwdArgs& a, hipStream_t s, int which) {
  constexpr int64_t kWavesPerBlock = kvc::kBwdThreads / kvc::kWave;
  // the statistics pass holds 4 rows a wave: 8-row heads take two waves a run
  constexpr int RG = ROWS / 4;
  const int64_t runs =
      which == 2 ? (a.M + kvc::kBwdSlotPassSlots - 1) / kvc::kBwdSlotPassSlots
                 : a.nchunk * (which == 0 ? RG : 1);
  const unsigned blocks =
      static_cast<unsigned>((a.B * a.Hk * runs + kWavesPerBlock - 1) / kWavesPerBlock);
  if (which == 0)
    hipLaunchKernelGGL((kvc::bwd_vstats_kernel<D, 4, RG>), dim3(blocks), dim3(kvc::kBwdThreads), 0,
                       s, a);
  else if (which == 1)
    hipLaunchKernelGGL((kvc::bwd_vdq_kernel<D, ROWS>), dim3(blocks), dim3(kvc::kBwdThreads), 0, s, a);
  else
    hipLaunchKernelGGL((kvc::bwd_vslot_kernel<D, ROWS>), dim3(blocks), dim3(kvc::kBwdThreads), 0, s, a);
}
// The generic kernels of kvc_backward_generic.h: any head sizes with
// D + Dv <= kBwdGenAccDoubles, any element-aligned buffers.
template <typename T>
void launch_bwd_generic(const kvc::BwdArgs& a, hipStream_t s, int which) {
  const dim3 grid(static_cast<unsigned>(a.B * a.Hk * a.nchunk)), block(kvc::kBwdThreads);
  if (which == 0)
    hipLaunchKernelGGL((kvc::bwd_gstats_kernel<T>), grid, block, 0, s, a);
  else if (which == 1)
    hipLaunchKernelGGL((kvc::bwd_gchunk_kernel<T>), grid, block,
                       static_cast<size_t>(a.gen_slots) * (a.D + a.Dv) * sizeof(double), s, a);
  else
    hipLaunchKernelGGL((kvc::bwd_gdq_kernel<T>), dim3(static_cast<unsigned>(a.B * a.Hq * a.Q)),
                       block, 0, s, a);
}
bool bwd_vec_ok(const kvc_dims* d, int dtype) {
  const int64_t R = (d->Hq / d->Hk) * d->Q;
  return dtype == KVC_BF16 && d->D == d->Dv && (d->D == 64 || d->D == 128) &&
         R <= kvc::kBwdVecRows;
}

const BwdEntry* find_bwd(const kvc_dims* d, int dtype) {
  for (const BwdEntry& e : kBwdTable)
    if (e.dtype == dtype && e.D == d->D && e.Dv == d->Dv) return &e;
  return nullptr;
}

bool bwd_vec_ok(const kvc_dims* d, int dtype);
size_t bwd_workspace(const kvc_dims* d, int dtype) {
  const size_t B = d->B, Hq = d->Hq, Hk = d->Hk, Q = d->Q, D = d->D, M = d->M;
  const size_t R = (d->Hq / d->Hk) * d->Q;
  const size_t nchunk = (d->M + kvc::kBwdSlots - 1) / kvc::kBwdSlots;
  const size_t sdp = bwd_vec_ok(d, dtype) ? align_up(B * Hk * R * M * 2 * 4, 256) : 0;
  return align_up(B * Hq * Q * 4 * 8, 256) + align_up(B * Hk * nchunk * R * 4 * 8, 256) +
         align_up(B * Hk * nchunk * R * D * 8, 256) + sdp;
}

}  // namespace

extern "C" {

size_t kvc_backward_workspace_bytes(const kvc_dims* dims, int dtype) {
  if (!dims || check_dims(dims, dtype) != KVC_OK) return 0;
  return bwd_workspace(dims, dtype);
}

int kvc_step_backward(const kvc_dims* dims, int dtype, int has_scale, double scale,
                      const void* query, const void* new_key, const void* new_value,
                      const void* key_cache, const void* value_cache, const int64_t* lengths,
                      const uint8_t* append_mask, const void* d_attention, const void* d_context,
                      const void* d_key_cache_out, const void* d_value_cache_out,
                      void* g_query, void* g_new_key, void* g_new_value, void* g_key_cache,
                      void* g_value_cache, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!dims) return KVC_ERR_NULL;
  const kvc_dims* d = dims;
  int rc = check_dims(d, dtype);
  if (rc != KVC_OK) return rc;
  const BwdEntry* e = find_bwd(d, dtype);
  if (!e && kvc::bwd_gen_slots(d->D, d->Dv) == 0) return KVC_ERR_UNSUPPORTED;
  double sc;
  rc = check_scale(has_scale, scale, d->D, &sc);
  if (rc != KVC_OK) return rc;
  if (!key_cache || !value_cache || !lengths || !g_key_cache || !g_value_cache || !workspace)
    return KVC_ERR_NULL;
  if (d->Q > 0 && (!query || !new_key || !new_value || !append_mask || !g_query || !g_new_key ||
                   !g_new_value))
    return KVC_ERR_NULL;
  // The tiled kernels move the K'/V', q and dO rows and the slot gradients
  // in 16-byte pieces; shapes without a tile, or buffers that are not
  // 16-byte aligned, take the generic kernels, which need each buffer
  // aligned to its element only.
  bool generic = !e;
  {
    const void* bufs[] = {key_cache, value_cache, d_key_cache_out, d_value_cache_out, g_key_cache,
                          g_value_cache, query, new_key, new_value, d_context, g_new_key,
                          g_new_value, d_attention, g_query};
    const uintptr_t el = dtype == KVC_BF16 ? 2u : 4u;
    for (const void* p : bufs) {
      const uintptr_t u = reinterpret_cast<uintptr_t>(p);
      if (u % el) return KVC_ERR_UNSUPPORTED;
      if (p != d_attention && p != g_query && (u & 15u)) generic = true;
    }
    if (generic && kvc::bwd_gen_slots(d->D, d->Dv) == 0) return KVC_ERR_UNSUPPORTED;
  }
  if (workspace_bytes < bwd_workspace(d, dtype)) return KVC_ERR_WORKSPACE;
  const size_t B = d->B, Hq = d->Hq, Hk = d->Hk, Q = d->Q, M = d->M, D = d->D, Dv = d->Dv;
  const size_t e4 = dtype == KVC_BF16 ? 2 : 4;  // element bytes
  const Range ins[] = {{query, B * Hq * Q * D * e4}, {new_key, B * Hk * Q * D * e4},
                       {new_value, B * Hk * Q * Dv * e4}, {key_cache, B * Hk * M * D * e4},
                       {value_cache, B * Hk * M * Dv * e4}, {lengths, B * 8},
                       {append_mask, B * Q}, {d_attention, B * Hq * Q * M * e4},
                       {d_context, B * Hq * Q * Dv * e4}, {d_key_cache_out, B * Hk * M * D * e4},
                       {d_value_cache_out, B * Hk * M * Dv * e4}};
  const Range outs[] = {{g_query, B * Hq * Q * D * e4}, {g_new_key, B * Hk * Q * D * e4},
                        {g_new_value, B * Hk * Q * Dv * e4}, {g_key_cache, B * Hk * M * D * e4},
                        {g_value_cache, B * Hk * M * Dv * e4}, {workspace, bwd_workspace(d, dtype)}};
  for (int i = 0; i < 6; i++) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return KVC_ERR_ALIAS;
    for (int j = i + 1; j < 6; j++)
      if (overlap(outs[i], outs[j])) return KVC_ERR_ALIAS;
  }
  (void)hipGetLastError();  // an earlier error is not ours
  kvc::BwdArgs a;
  std::memset(&a, 0, sizeof a);
  a.B = d->B; a.Hq = d->Hq; a.Hk = d->Hk; a.Q = d->Q; a.M = d->M; a.D = d->D; a.Dv = d->Dv;
  a.G = static_cast<int32_t>(d->Hq / d->Hk);
  a.R = static_cast<int32_t>(a.G * d->Q);
  const bool vec = !generic && bwd_vec_ok(d, dtype);
  a.part_slots = vec ? kvc::kBwdVecSlots : kvc::kBwdSlots;
  a.nchunk = (d->M + a.part_slots - 1) / a.part_slots;
  {
    const int64_t tiles = (a.R + kvc::kBwdRowTile - 1) / kvc::kBwdRowTile;
    a.row_groups = static_cast<int32_t>(tiles < 1 ? 1 : tiles < kvc::kBwdMaxRowGroups ? tiles : kvc::kBwdMaxRowGroups);
  }
  {  // every grid must fit one launch: the chunk grids (chunks x row or
     // column groups) and the per-row grids (one row per workgroup for dq)
    int64_t x;
    if (!mul_ok(d->B * d->Hk, a.nchunk, kMaxElems, &x) ||
        !mul_ok(x, a.row_groups > 4 ? a.row_groups : 4, kMaxBwdWorkgroups, &x) ||
        !mul_ok(d->B * d->Hq, d->Q, kMaxElems, &x) || x > kMaxBwdWorkgroups)
      return KVC_ERR_SHAPE;
  }
  a.scale = static_cast<float>(sc);
  a.scale_d = sc;
  a.gen_slots = generic ? kvc::bwd_gen_slots(d->D, d->Dv) : 0;
  a.query = query;
  a.new_key = new_key;
  a.new_value = new_value;
  a.kc = key_cache;
  a.vc = value_cache;
  a.lengths = lengths;
  a.mask = append_mask;
  a.d_att = d_attention;
  a.d_ctx = d_context;
  a.d_kc_out = d_key_cache_out;
  a.d_vc_out = d_value_cache_out;
  a.g_query = g_query;
  a.g_new_key = g_new_key;
  a.g_new_value = g_new_value;
  a.g_kc = g_key_cache;
  a.g_vc = g_value_cache;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const size_t nchunk = static_cast<size_t>(a.nchunk), R = static_cast<size_t>(a.R);
  a.ws_row = reinterpret_cast<double*>(ws);
  a.ws_part = reinterpret_cast<double*>(ws + align_up(B * Hq * Q * 4 * 8, 256));
  a.ws_dq = reinterpret_cast<double*>(ws + align_up(B * Hq * Q * 4 * 8, 256) +
                                      align_up(B * Hk * nchunk * R * 4 * 8, 256));
  {  // after the partial arrays at their largest (64-slot chunks)
    const size_t n64 = (d->M + kvc::kBwdSlots - 1) / kvc::kBwdSlots;
    a.ws_sdp = reinterpret_cast<float*>(ws + align_up(B * Hq * Q * 4 * 8, 256) +
                                        align_up(B * Hk * n64 * R * 4 * 8, 256) +
                                        align_up(B * Hk * n64 * R * D * 8, 256));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows = d->B * d->Hq * d->Q;
  const unsigned row_blocks = static_cast<unsigned>((rows + 3) / 4);
  if (generic) {  // statistics, rows, chunks (dq partials, slot gradients), dq
    auto run = [&](int which) {
      dtype == KVC_BF16 ? launch_bwd_generic<kvc::bf16>(a, s, which)
                        : launch_bwd_generic<float>(a, s, which);
    };
    if (rows > 0) {
      run(0);
      hipLaunchKernelGGL(kvc::bwd_rows_kernel, dim3(row_blocks), dim3(kvc::kBwdThreads), 0, s, a);
    }
    run(1);
    if (rows > 0) run(2);
    return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
  }
  if (vec) {  // statistics, rows, dq partials, slot gradients, dq
    auto run = [&](int which) {
      if (a.R <= 4)
        d->D == 128 ? launch_bwd_vec<128, 4>(a, s, which) : launch_bwd_vec<64, 4>(a, s, which);
      else
        d->D == 128 ? launch_bwd_vec<128, 8>(a, s, which) : launch_bwd_vec<64, 8>(a, s, which);
    };
    if (rows > 0) {
      run(0);
      hipLaunchKernelGGL(kvc::bwd_rows_kernel, dim3(row_blocks), dim3(kvc::kBwdThreads), 0, s, a);
      run(1);
    }
    run(2);
    if (rows > 0) e->dq(a, s);
    return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
  }
  if (rows > 0) {
    e->stats(a, s);
    hipLaunchKernelGGL(kvc::bwd_rows_kernel, dim3(row_blocks), dim3(kvc::kBwdThreads), 0, s, a);
  }
  e->chunk(a, s);
  if (rows > 0) e->dq(a, s);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

}  // extern "C"
