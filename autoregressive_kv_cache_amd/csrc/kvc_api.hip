// kvc_api.hip -- host side of the C ABI declared in include/kvc.h: argument
// checks, kernel plan, workspace layout and launches on the caller's stream.
// No allocation, no synchronisation, no state kept between calls.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/kvc.h"
#include "kvc_chunk.h"
#include "kvc_combine.h"
#include "kvc_common.h"
#include "kvc_decode.h"
#include "kvc_generic.h"
#include "kvc_host.h"
#include "kvc_prep.h"
#include "kvc_reattend.h"
#include "kvc_combine_stream.h"
#include "kvc_small.h"
#include "kvc_stream.h"

namespace {

using kvc::StepArgs;
using namespace kvc_host;

constexpr int64_t kMaxWorkgroups = int64_t(1) << 24;


// Vector decode kernels compiled in: (dtype, D, Dv, packed rows).
template <typename T, int D, int DV, int ROWS, bool Q1>
void launch_decode_q(const StepArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.P / kvc::kDecodeWaves)), block(kvc::kDecodeThreads);
  const int64_t* ri = a.ws_rowinfo;
  const int32_t* wst = a.ws_wstart;
  const bool fused = a.B <= kvc::kDecodeFusedRows;
  if (a.paged && fused)
    hipLaunchKernelGGL((kvc::attend_decode_kernel<T, D, DV, ROWS, Q1, false, true, true>), grid,
                       block, 0, s, a, ri, wst);
  else if (a.paged)
    hipLaunchKernelGGL((kvc::attend_decode_kernel<T, D, DV, ROWS, Q1, false, false, true>), grid,
                       block, 0, s, a, ri, wst);
  else if (a.out_of_place && fused)
    hipLaunchKernelGGL((kvc::attend_decode_kernel<T, D, DV, ROWS, Q1, true, true, false>), grid,
                       block, 0, s, a, ri, wst);
  else if (a.out_of_place)
    hipLaunchKernelGGL((kvc::attend_decode_kernel<T, D, DV, ROWS, Q1, true, false, false>), grid,
                       block, 0, s, a, ri, wst);
  else if (fused)
    hipLaunchKernelGGL((kvc::attend_decode_kernel<T, D, DV, ROWS, Q1, false, true, false>), grid,
                       block, 0, s, a, ri, wst);
  else
    hipLaunchKernelGGL((kvc::attend_decode_kernel<T, D, DV, ROWS, Q1, false, false, false>), grid,
                       block, 0, s, a, ri, wst);
}

template <typename T, int D, int DV, int ROWS>
void launch_decode(const StepArgs& a, hipStream_t s) {
  if (a.Q == 1)
    launch_decode_q<T, D, DV, ROWS, true>(a, s);
  else
    launch_decode_q<T, D, DV, ROWS, false>(a, s);
}

// bf16 caches: the stream kernel of kvc_stream.h.
template <int D, int DV, int ROWS, bool Q1, bool G>
void launch_stream_g(const StepArgs& a, hipStream_t s) {
  // rg_waves waves per stream worker
  const dim3 grid(static_cast<unsigned>(a.P * a.rg_waves / kvc::kDecodeWaves)),
      block(kvc::kDecodeThreads);
  const int64_t* ri = a.ws_rowinfo;
  const int32_t* wst = a.ws_wstart;
  const bool fused = a.B <= kvc::kDecodeFusedRows;
  if (a.paged && fused)
    hipLaunchKernelGGL((kvc::attend_stream_kernel<D, DV, ROWS, Q1, false, true, true, G>), grid,
                       block, 0, s, a, ri, wst);
  else if (a.paged)
    hipLaunchKernelGGL((kvc::attend_stream_kernel<D, DV, ROWS, Q1, false, false, true, G>), grid,
                       block, 0, s, a, ri, wst);
  else if (a.out_of_place && fused)
    hipLaunchKernelGGL((kvc::attend_stream_kernel<D, DV, ROWS, Q1, true, true, false, G>), grid,
                       block, 0, s, a, ri, wst);
  else if (a.out_of_place)
    hipLaunchKernelGGL((kvc::attend_stream_kernel<D, DV, ROWS, Q1, true, false, false, G>), grid,
                       block, 0, s, a, ri, wst);
  else if (fused)
    hipLaunchKernelGGL((kvc::attend_stream_kernel<D, DV, ROWS, Q1, false, true, false, G>), grid,
                       block, 0, s, a, ri, wst);
  else
    hipLaunchKernelGGL((kvc::attend_stream_kernel<D, DV, ROWS, Q1, false, false, false, G>), grid,
                       block, 0, s, a, ri, wst);
}

template <int D, int DV, int ROWS, bool Q1>
void launch_stream_q(const StepArgs& a, hipStream_t s) {
  if constexpr (ROWS == 8) {  // row groups: past 8 packed rows only
    if (a.rg_waves > 1) {
      launch_stream_g<D, DV, ROWS, Q1, true>(a, s);
      return;
    }
  }
  launch_stream_g<D, DV, ROWS, Q1, false>(a, s);
}

template <typename T, int D, int DV, int ROWS>
void launch_decode_bf16(const StepArgs& a, hipStream_t s) {
  if (a.Q == 1)
    launch_stream_q<D, DV, ROWS, true>(a, s);
  else
    launch_stream_q<D, DV, ROWS, false>(a, s);
}

// Small heads (rows of at most 64 bytes): the one-slot-per-lane kernel of
// kvc_small.h, one launch for every variant (the row table, the paged
// source and the out-of-place copy are chosen at run time).
template <typename T, int D, int DV, int ROWS>
void launch_small(const StepArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.P / kvc::kDecodeWaves)), block(kvc::kDecodeThreads);
  hipLaunchKernelGGL((kvc::attend_small_kernel<T, D, DV, ROWS>), grid, block, 0, s, a,
                     a.ws_rowinfo, a.ws_wstart);
}

struct DecodeEntry {
  int dtype, D, Dv, rows, chunk, wgs_per_cu;
  void (*launch)(const StepArgs&, hipStream_t);
  bool stream;  // attend_stream_kernel (its own workspace layout and combine)
  int lead;     // share weight of the first half of the workers, in eighths (8: even)
};

#define KVC_DECODE(T, CODE, D, DV, ROWS) \
  {CODE, D, DV, ROWS, kvc::decode_chunk<T, D, DV, ROWS>(), kvc::decode_waves_per_simd<ROWS>(), \
   &launch_decode<T, D, DV, ROWS>, false, 8}
// the two kernels of a bf16 entry share chunk size and occupancy.  Were a
// unit to hold two stream workgroups, the first one placed would take twice
// the share (its waves win the SIMDs' issue arbitration; measured 2.3 us
// less per decode step at B=32, Hq=32, Hk=8, M=8192 than even shares); the
// stream entries now hold one workgroup per unit, and even shares.
#define KVC_SMALL(T, CODE, D, DV, ROWS) \
  {CODE, D, DV, ROWS, kvc::kSmallChunk, 2, &launch_small<T, D, DV, ROWS>, false, 8}
#define KVC_STREAM(D, DV, ROWS) \
  {KVC_BF16, D, DV, ROWS, kvc::kStreamChunk, kvc::stream_waves_per_simd<ROWS>(), \
   &launch_decode_bf16<kvc::bf16, D, DV, ROWS>, true, \
   kvc::stream_waves_per_simd<ROWS>() == 2 ? 16 : 8}
const DecodeEntry kDecodeTable[] = {
    KVC_STREAM(128, 128, 4), KVC_STREAM(128, 128, 8), KVC_STREAM(64, 64, 4), KVC_STREAM(64, 64, 8),
    KVC_DECODE(kvc::bf16, KVC_BF16, 256, 256, 4), KVC_DECODE(kvc::bf16, KVC_BF16, 256, 256, 8),
    KVC_DECODE(float, KVC_F32, 128, 128, 4),      KVC_DECODE(float, KVC_F32, 64, 64, 4),
    KVC_DECODE(float, KVC_F32, 64, 32, 4),
    KVC_SMALL(float, KVC_F32, 8, 8, 4),           KVC_SMALL(float, KVC_F32, 8, 8, 8),
    KVC_SMALL(float, KVC_F32, 16, 16, 4),         KVC_SMALL(float, KVC_F32, 16, 16, 8),
    KVC_SMALL(kvc::bf16, KVC_BF16, 16, 16, 4),    KVC_SMALL(kvc::bf16, KVC_BF16, 16, 16, 8),
    KVC_SMALL(kvc::bf16, KVC_BF16, 32, 32, 4),    KVC_SMALL(kvc::bf16, KVC_BF16, 32, 32, 8),
};
#undef KVC_SMALL
#undef KVC_DECODE
#undef KVC_STREAM

// Stream path: every compute unit of the current device holds as many attend
// workgroups (of 4 waves, one per SIMD, each wave one stream worker) as the
// kernel's registers allow, and each wave keeps a whole chunk of loads in
// flight.  The count comes from the device (256 on MI355X); without a device
// (a host-only caller) the MI355X count is assumed.
int64_t compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}
// Slots per combine workgroup (a multiple of every chunk size).  Out of
// place the combine also copies the cache slots the attend kernel did not
// visit, and more, narrower ranges spread that copy over more workgroups:
// 512 slots took the long decode's out-of-place step from 1026 to 929 us
// and the decode one from 467 to 451 us against 4096 (1024 and 256 were
// between).
constexpr int64_t kCombineSlots = 4096;
constexpr int64_t kCombineSlotsCopy = 512;

// Matrix-core chunk path: kChunkMinRows (16) packed rows per KV head or more.
struct ChunkEntry {
  int dtype;
  int64_t D, Dv;
  void (*launch)(const StepArgs&, hipStream_t);
};

template <int D, int DV>
void launch_chunk(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((kvc::attend_chunk_kernel<D, DV>),
                     dim3(static_cast<unsigned>(a.B * a.Hk * a.nchunk_max *
                                                kvc::chunk_row_groups(a.R))),
                     dim3(kvc::kChunkThreads), 0, s, a);
}

template <int D, int DV>
void launch_chunk_f32(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((kvc::attend_chunk_f32_kernel<D, DV>),
                     dim3(static_cast<unsigned>(a.B * a.Hk * a.nchunk_max *
                                                kvc::chunk_row_groups(a.R))),
                     dim3(kvc::kChunkThreads), 0, s, a);
}

// bf16 on the bf16 matrix cores, fp32 on the fp64 ones
const ChunkEntry kChunkTable[] = {
    {KVC_BF16, 64, 64, &launch_chunk<64, 64>},
    {KVC_BF16, 128, 128, &launch_chunk<128, 128>},
    {KVC_BF16, 256, 256, &launch_chunk<256, 256>},
    {KVC_F32, 64, 64, &launch_chunk_f32<64, 64>},
    {KVC_F32, 128, 128, &launch_chunk_f32<128, 128>},
};

// The matrix-core chunk path: only where the packed rows of a KV head fill
// at least one 16-row MFMA tile ("a real dense contraction").
constexpr int64_t kChunkMinRows = 16;
const ChunkEntry* find_chunk(const kvc_dims* d, int dtype, int64_t R) {
  if (R < kChunkMinRows) return nullptr;
  for (const ChunkEntry& e : kChunkTable)
    if (e.dtype == dtype && e.D == d->D && e.Dv == d->Dv) return &e;
  return nullptr;
}

// The vector decode path: a wave holds 4 or 8 packed rows.  Past 8 (up to
// 15: the chunk path starts at 16) the bf16 stream kernel splits the rows
// into two groups of up to 8, two waves of one worker (*rg_waves = 2).
constexpr int64_t kStreamMaxRows = kChunkMinRows - 1;
const DecodeEntry* find_decode(const kvc_dims* d, int dtype, int64_t R, int* rg_waves) {
  *rg_waves = 1;
  const int rows = R <= 4 ? 4 : 8;
  for (const DecodeEntry& e : kDecodeTable) {
    if (e.dtype != dtype || e.D != d->D || e.Dv != d->Dv || e.rows != rows) continue;
    if (R <= 8) return &e;
    if (e.stream && R <= kStreamMaxRows) {
      *rg_waves = 2;
      return &e;
    }
  }
  return nullptr;
}

struct Layout {
  int64_t C, nchunk_max, nseg, CS;
  size_t off_hdr, off_rowinfo, off_chunk, off_seg_ml, off_seg_o, off_wstart, off_pexp, off_cref,
      off_seg2, bytes;
};

// stream2: the arrays of attend_stream_kernel (exp values and references
// per chunk, segment statistics in float) instead of the per-chunk double
// statistics of the other attend kernels.
bool make_layout(const kvc_dims* d, int64_t R, int64_t C, bool stream,
                 int64_t P, Layout* L, bool stream2 = false) {
  L->C = C;
  // stream mode: the cached slots in chunks of C plus one chunk of the
  // appended rows per head
  L->nchunk_max = (d->M + C - 1) / C + (stream ? 1 : 0);
  L->CS = kCombineSlots;
  int64_t groups, chunks, nseg, x;
  if (!mul_ok(d->B, d->Hk, kMaxElems, &groups) || !mul_ok(groups, L->nchunk_max, kMaxElems, &chunks))
    return false;
  nseg = stream ? P + groups : chunks;
  L->nseg = nseg;
  size_t off = 0;
  L->off_hdr = off;
  off = align_up(off + 8 * sizeof(int64_t), 256);
  L->off_rowinfo = off;
  off = align_up(off + static_cast<size_t>(d->B) * 4 * sizeof(int64_t), 256);
  L->off_chunk = off;
  if (!mul_ok(chunks, R, kMaxElems, &x)) return false;
  if (!stream2) off = align_up(off + static_cast<size_t>(x) * 2 * sizeof(double), 256);
  L->off_seg_ml = off;
  if (!mul_ok(nseg, R, kMaxElems, &x)) return false;
  off = align_up(off + static_cast<size_t>(x) * 2 * sizeof(double), 256);
  L->off_seg_o = off;
  if (!mul_ok(x, d->Dv, kMaxElems, &x)) return false;
  off = align_up(off + static_cast<size_t>(x) * sizeof(float), 256);
  L->off_wstart = off;
  off = align_up(off + static_cast<size_t>(stream ? P : 0) * 4 * sizeof(int32_t), 256);
  L->off_pexp = L->off_cref = L->off_seg2 = off;
  if (stream2) {
    int64_t xr;  // chunks x rows
    if (!mul_ok(chunks, R, kMaxElems, &xr) || !mul_ok(xr, C, kMaxElems, &x)) return false;
    L->off_pexp = off;
    off = align_up(off + static_cast<size_t>(x) * sizeof(uint16_t), 256);
    L->off_cref = off;
    off = align_up(off + static_cast<size_t>(xr) * sizeof(float), 256);
    if (!mul_ok(nseg, R, kMaxElems, &x)) return false;
    L->off_seg2 = off;
    off = align_up(off + static_cast<size_t>(x) * 2 * sizeof(float), 256);
  }
  L->bytes = off;
  return true;
}

struct Plan {
  kvc_plan pub;
  const DecodeEntry* decode;  // vector decode path, or null
  const ChunkEntry* chunk;    // matrix-core chunk path, or null
  Layout generic, stream, dense;
  int64_t P;     // stream workers
  int rg_waves;  // waves per stream worker
};

int make_plan(const kvc_dims* d, int dtype, Plan* p) {
  int rc = check_dims(d, dtype);
  if (rc != KVC_OK) return rc;
  std::memset(p, 0, sizeof *p);
  const int64_t R = (d->Hq / d->Hk) * d->Q;
  p->pub.rows = static_cast<int32_t>(R);
  p->decode = find_decode(d, dtype, R, &p->rg_waves);
  p->chunk = p->decode ? nullptr : find_chunk(d, dtype, R);
  p->P = p->decode
             ? compute_units() * p->decode->wgs_per_cu * (kvc::kDecodeWaves / p->rg_waves)
             : 0;
  if (p->decode) {
    // no more workers than the step can have chunks (every (b, KV head):
    // its cached slots in chunks, plus one chunk of appended rows), rounded
    // to whole workgroups: small steps launch a few workgroups, not a full
    // grid of idle ones.  Busy workers are min(P, chunks) either way.
    const int64_t most = d->B * d->Hk * ((d->M + p->decode->chunk - 1) / p->decode->chunk + 1);
    const int64_t cap = (most + kvc::kDecodeWaves - 1) / kvc::kDecodeWaves * kvc::kDecodeWaves;
    if (p->P > cap) p->P = cap;
  }
  const int64_t row_tiles = R == 0 ? 1 : (R + kvc::kGenericRowsPerTile - 1) / kvc::kGenericRowsPerTile;
  if (!make_layout(d, R, kvc::kGenericChunk, false, 0, &p->generic)) return KVC_ERR_SHAPE;
  int64_t wgs;
  // combine grid: groups x (slot ranges + 1) x blocks of kCombineWaves rows
  const int64_t row_blocks = R == 0 ? 1 : (R + kvc::kCombineWaves - 1) / kvc::kCombineWaves;
  if (!mul_ok(d->B * d->Hk, row_tiles, kMaxElems, &wgs) ||
      !mul_ok(wgs, p->generic.nchunk_max, kMaxWorkgroups, &wgs) ||
      !mul_ok(d->B * d->Hk, row_blocks, kMaxElems, &wgs) ||
      !mul_ok(wgs, (d->M + kCombineSlotsCopy - 1) / kCombineSlotsCopy + 1, kMaxWorkgroups, &wgs))
    return KVC_ERR_SHAPE;
  size_t bytes = p->generic.bytes;
  if (p->decode) {
    if (!make_layout(d, R, p->decode->chunk, true, p->P, &p->stream, p->decode->stream))
      return KVC_ERR_SHAPE;
    int64_t cwgs;
    if (!mul_ok(d->B * d->Hk, row_blocks, kMaxElems, &cwgs) ||
        !mul_ok(cwgs, (d->M + kCombineSlotsCopy - 1) / kCombineSlotsCopy + 1, kMaxWorkgroups, &cwgs))
      return KVC_ERR_SHAPE;
    if (p->stream.bytes > bytes) bytes = p->stream.bytes;
    p->pub.path = 1;
    p->pub.rows_per_tile = p->decode->rows;
    p->pub.row_tiles = static_cast<int32_t>(R <= p->decode->rows ? 1 : (R + p->decode->rows - 1) /
                                                                        p->decode->rows);
    p->pub.split = p->decode->chunk;
    p->pub.nsplit = p->stream.nchunk_max;
    p->pub.workers = p->P;
    p->pub.lead = p->decode->lead;
  } else if (p->chunk) {
    if (!make_layout(d, R, kvc::kChunkSlots, false, 0, &p->dense)) return KVC_ERR_SHAPE;
    int64_t cwgs;
    if (!mul_ok(d->B * d->Hk, p->dense.nchunk_max * kvc::chunk_row_groups(R), kMaxWorkgroups,
                &cwgs) ||
        !mul_ok(d->B * d->Hk, row_blocks, kMaxElems, &cwgs) ||
        !mul_ok(cwgs, (d->M + kCombineSlotsCopy - 1) / kCombineSlotsCopy + 1, kMaxWorkgroups, &cwgs))
      return KVC_ERR_SHAPE;
    if (p->dense.bytes > bytes) bytes = p->dense.bytes;
    p->pub.path = 2;
    p->pub.rows_per_tile = static_cast<int32_t>(R);
    p->pub.row_tiles = 1;
    p->pub.split = kvc::kChunkSlots;
    p->pub.nsplit = p->dense.nchunk_max;
  } else {
    p->pub.path = 0;
    p->pub.rows_per_tile = kvc::kGenericRowsPerTile;
    p->pub.row_tiles = static_cast<int32_t>(row_tiles);
    p->pub.split = kvc::kGenericChunk;
    p->pub.nsplit = p->generic.nchunk_max;
  }
  p->pub.workspace_bytes = bytes;
  return KVC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void set_layout(StepArgs& a, const Layout& L, void* workspace) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.C = L.C;
  a.C_log2 = 0;
  while ((int64_t(1) << a.C_log2) < L.C) a.C_log2++;
  a.nchunk_max = L.nchunk_max;
  a.CS = a.out_of_place ? kCombineSlotsCopy : L.CS;
  a.ws_hdr = reinterpret_cast<int64_t*>(ws + L.off_hdr);
  a.ws_rowinfo = reinterpret_cast<int64_t*>(ws + L.off_rowinfo);
  a.ws_chunk_ml = reinterpret_cast<double*>(ws + L.off_chunk);
  a.ws_seg_ml = reinterpret_cast<double*>(ws + L.off_seg_ml);
  a.ws_seg_o = reinterpret_cast<float*>(ws + L.off_seg_o);
  a.ws_wstart = reinterpret_cast<int32_t*>(ws + L.off_wstart);
  a.ws_pexp = reinterpret_cast<uint16_t*>(ws + L.off_pexp);
  a.ws_cref = reinterpret_cast<float*>(ws + L.off_cref);
  a.ws_seg2 = reinterpret_cast<float*>(ws + L.off_seg2);
}

template <typename T>
void launch_combine(const StepArgs& a, hipStream_t stream) {
  const int64_t groups = a.B * a.Hk;
  const int64_t nrb = a.R > 0 ? (a.R + kvc::kCombineWaves - 1) / kvc::kCombineWaves : 1;
  const int64_t roles = a.read_only ? 1 : (a.M + a.CS - 1) / a.CS + 1;
  hipLaunchKernelGGL(kvc::combine_kernel<T>, dim3(static_cast<unsigned>(groups * roles * nrb)),
                     dim3(kvc::kCombineThreads), 0, stream, a);
}

template <typename T>
void launch_generic(StepArgs& a, hipStream_t stream, const kvc_events* ev) {
  const int64_t groups = a.B * a.Hk;
  if (ev && ev->start) hipEventRecord(static_cast<hipEvent_t>(ev->start), stream);
  hipLaunchKernelGGL(kvc::attend_generic_kernel<T>,
                     dim3(static_cast<unsigned>(groups * a.row_tiles * a.nchunk_max)),
                     dim3(kvc::kGenericThreads), 0, stream, a);
  if (ev && ev->stop) hipEventRecord(static_cast<hipEvent_t>(ev->stop), stream);
  launch_combine<T>(a, stream);
}

void launch_dense_chunk(StepArgs& a, const ChunkEntry& e, hipStream_t stream,
                        const kvc_events* ev) {
  if (ev && ev->start) hipEventRecord(static_cast<hipEvent_t>(ev->start), stream);
  e.launch(a, stream);
  if (ev && ev->stop) hipEventRecord(static_cast<hipEvent_t>(ev->stop), stream);
  if (e.dtype == KVC_F32)
    launch_combine<float>(a, stream);
  else
    launch_combine<kvc::bf16>(a, stream);
}

template <typename T>
void launch_stream(StepArgs& a, const DecodeEntry& e, hipStream_t stream, const kvc_events* ev) {
  const int64_t groups = a.B * a.Hk;
  // up to kDecodeFusedRows rows the attend kernel prepares the rows itself
  if (a.B > kvc::kDecodeFusedRows)
    hipLaunchKernelGGL(kvc::prep_kernel, dim3(1), dim3(kvc::kPrepThreads), 0, stream, a);
  if (ev && ev->start) hipEventRecord(static_cast<hipEvent_t>(ev->start), stream);
  e.launch(a, stream);
  if (ev && ev->stop) hipEventRecord(static_cast<hipEvent_t>(ev->stop), stream);
  if (e.stream) {
    const int64_t groups = a.B * a.Hk;
    const int64_t nrb = a.R > 0 ? (a.R + kvc::kCombineWaves - 1) / kvc::kCombineWaves : 1;
    const int64_t roles = a.read_only ? 1 : (a.M + a.CS - 1) / a.CS + 1;
    hipLaunchKernelGGL(kvc::combine_stream_kernel, dim3(static_cast<unsigned>(groups * roles * nrb)),
                       dim3(kvc::kCombineThreads), 0, stream, a);
  } else {
    launch_combine<T>(a, stream);
  }
}

// The paged layout: block pools [num_blocks][Hk][block_size][D or Dv] and a
// [B][M / block_size] int32 block table.
struct PagedPool {
  int64_t num_blocks, block_size;
  const int32_t* table;  // [B][M / block_size], or none with identity (block b)
  bool identity;
};

void set_paged(StepArgs& a, const kvc_dims* d, const PagedPool& pg) {
  a.paged = 1;
  a.num_blocks = pg.num_blocks;
  a.max_blocks = d->M / pg.block_size;
  a.block_table = pg.table;
  a.block_rows = pg.block_size;
  a.block_log2 = 0;
  if (pg.block_size == d->M) {  // one block per row (any M)
    a.block_log2 = 62;
    a.block_mask = -1;
  } else {
    while ((int64_t(1) << a.block_log2) < pg.block_size) a.block_log2++;
    a.block_mask = pg.block_size - 1;
  }
}

int run_step(const kvc_dims* d, int dtype, int has_scale, double scale, const void* query,
             const void* new_key, const void* new_value, const void* kc_in, const void* vc_in,
             void* kc_out, void* vc_out, bool out_of_place, const int64_t* lengths,
             const uint8_t* mask, int64_t* lengths_out, void* attention, void* context,
             int32_t* row_status, void* workspace, size_t workspace_bytes, void* stream,
             const kvc_events* events, const PagedPool* pg = nullptr, bool read_only = false,
             const float* sinks = nullptr) {
  Plan p;
  int rc = make_plan(d, dtype, &p);
  if (rc != KVC_OK) return rc;
  double sc;
  rc = check_scale(has_scale, scale, d->D, &sc);
  if (rc != KVC_OK) return rc;

  if (pg) {
    if (!pg->table && !pg->identity) return KVC_ERR_NULL;
    const int64_t bs = pg->block_size;
    const bool single = bs == d->M;  // one block per row: a continuous cache, rows by table
    if (pg->num_blocks < 1 || bs < 1 || (!single && ((bs & (bs - 1)) != 0 || d->M % bs != 0)))
      return KVC_ERR_SHAPE;
    int64_t x;
    if (!mul_ok(pg->num_blocks, d->Hk, kMaxElems, &x) || !mul_ok(x, bs, kMaxElems, &x) ||
        !mul_ok(x, d->D > d->Dv ? d->D : d->Dv, kMaxElems, &x))
      return KVC_ERR_SHAPE;
  }

  if (!kc_in || !vc_in || !kc_out || !vc_out || !lengths || !lengths_out) return KVC_ERR_NULL;
  // (read-only re-attention writes no attention rows: none is passed)
  if (d->Q > 0 && (!query || !new_key || !new_value || !mask || (!attention && !read_only) ||
                   !context))
    return KVC_ERR_NULL;
  if (p.pub.workspace_bytes > 0 && !workspace) return KVC_ERR_NULL;
  if (workspace_bytes < p.pub.workspace_bytes) return KVC_ERR_WORKSPACE;

  const size_t e = dtype == KVC_F32 ? 4 : 2;
  const size_t B = d->B, Hq = d->Hq, Hk = d->Hk, Q = d->Q, M = d->M, D = d->D, Dv = d->Dv;
  // cache extent: B rows of M slots, or the block pools
  const size_t slots = pg ? static_cast<size_t>(pg->num_blocks * pg->block_size) : B * M;
  const Range r_q{query, B * Hq * Q * D * e}, r_nk{new_key, B * Hk * Q * D * e},
      r_nv{new_value, B * Hk * Q * Dv * e}, r_kin{kc_in, Hk * slots * D * e},
      r_vin{vc_in, Hk * slots * Dv * e}, r_len{lengths, B * 8}, r_mask{mask, B * Q},
      r_kout{kc_out, Hk * slots * D * e}, r_vout{vc_out, Hk * slots * Dv * e},
      r_lout{lengths_out, B * 8}, r_att{attention, B * Hq * Q * M * e},
      r_ctx{context, B * Hq * Q * Dv * e}, r_st{row_status, row_status ? B * 4 : 0},
      r_ws{workspace, p.pub.workspace_bytes};
  const Range r_tab{pg ? pg->table : nullptr, pg && pg->table ? B * (M / pg->block_size) * 4 : 0};
  const bool len_in_place = !out_of_place && lengths_out == lengths;
  const Range inputs[] = {r_q, r_nk, r_nv, r_mask, r_tab,
                          len_in_place ? Range{nullptr, 0} : r_len};
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
    const Range others[] = {r_q, r_nk, r_nv, r_mask, r_tab, r_kin, r_vin, r_att, r_ctx, r_st, r_ws};
    for (const Range& o : others)
      if (overlap(r_len, o)) return KVC_ERR_ALIAS;
  }
  if (!out_of_place) {  // the two caches are written in place
    for (const Range& in : inputs)
      for (const Range& c : caches_in)
        if (overlap(in, c)) return KVC_ERR_ALIAS;
    if (overlap(r_kin, r_vin)) return KVC_ERR_ALIAS;
  }

  // an error left by earlier, unrelated work must not be reported as ours
  (void)hipGetLastError();
  StepArgs a;
  std::memset(&a, 0, sizeof a);
  a.B = d->B; a.Hq = d->Hq; a.Hk = d->Hk; a.Q = d->Q; a.M = d->M; a.D = d->D; a.Dv = d->Dv;
  a.G = static_cast<int32_t>(d->Hq / d->Hk);
  a.R = p.pub.rows;
  a.rows_per_tile = p.pub.rows_per_tile;
  a.row_tiles = p.pub.row_tiles;
  a.P = p.P;
  a.rg_waves = p.rg_waves > 0 ? p.rg_waves : 1;
  a.lead = p.decode ? p.decode->lead : 8;
  a.scale = sc;
  a.elem_bytes = static_cast<int64_t>(e);
  a.out_of_place = out_of_place ? 1 : 0;
  a.query = query; a.new_key = new_key; a.new_value = new_value;
  a.kc_in = kc_in; a.vc_in = vc_in; a.kc_out = kc_out; a.vc_out = vc_out;
  a.lengths = lengths; a.mask = mask; a.attention = attention; a.context = context;
  a.lengths_out = lengths_out; a.row_status = row_status;

  // the vector and matrix paths need 16-byte aligned rows, and on a paged
  // cache every one of their chunks inside one block; other calls take the
  // generic kernel
  bool aligned = aligned16(query) && aligned16(new_key) && aligned16(new_value) &&
                 aligned16(kc_in) && aligned16(vc_in) && aligned16(kc_out) && aligned16(vc_out);
  if (pg) {
    const int64_t chunk = p.decode ? p.decode->chunk : (p.chunk ? kvc::kChunkSlots : 0);
    if (pg->block_size != d->M && pg->block_size < chunk) aligned = false;
    set_paged(a, d, *pg);
  }
  const bool vec_ok = p.decode && aligned;
  a.read_only = read_only ? 1 : 0;
  a.sinks = sinks;
  const bool chunk_ok = p.chunk && aligned;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (chunk_ok) {
    set_layout(a, p.dense, workspace);
    a.seg_mode = 0;
    a.combine_copies_tail = 0;
    a.rows_per_tile = a.R;
    a.row_tiles = 1;
    launch_dense_chunk(a, *p.chunk, s, events);
  } else if (vec_ok) {
    set_layout(a, p.stream, workspace);
    a.seg_mode = p.decode->stream ? 2 : 1;
    a.combine_copies_tail = 1;
    a.rows_per_tile = p.decode->rows;
    a.row_tiles = 1;
    if (dtype == KVC_F32)
      launch_stream<float>(a, *p.decode, s, events);
    else
      launch_stream<kvc::bf16>(a, *p.decode, s, events);
  } else {
    set_layout(a, p.generic, workspace);
    a.seg_mode = 0;
    a.combine_copies_tail = 0;
    a.rows_per_tile = kvc::kGenericRowsPerTile;
    a.row_tiles = static_cast<int32_t>(a.R == 0 ? 1 : (a.R + kvc::kGenericRowsPerTile - 1) /
                                                        kvc::kGenericRowsPerTile);
    if (dtype == KVC_F32)
      launch_generic<float>(a, s, events);
    else
      launch_generic<kvc::bf16>(a, s, events);
  }
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// Workspace of a re-attention: the equivalent step's own workspace, then its
// inputs (old lengths, mask, query rows, the appended-row copies) and
// outputs (lengths, status, attention, context).
// The equivalent step's inputs and context (no attention rows: the step runs
// read-only and writes none).
struct ReattLayout {
  size_t step, len0, lens_out, rstat, status, mask, qs, nk, nv, ctx, bytes;
};

bool reatt_layout(const kvc_dims* d, int dtype, ReattLayout* L) {
  Plan p;
  if (make_plan(d, dtype, &p) != KVC_OK) return false;
  const size_t e = dtype == KVC_F32 ? 4 : 2;
  const size_t B = d->B, Hq = d->Hq, Hk = d->Hk, Q = d->Q, M = d->M, D = d->D, Dv = d->Dv;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  L->step = p.pub.workspace_bytes;
  take(L->step);
  L->len0 = take(B * 8);
  L->lens_out = take(B * 8);
  L->rstat = take(B * 4);
  L->status = take(B * 4);
  L->mask = take(B * Q);
  L->qs = take(B * Hq * Q * D * e);
  L->nk = take(B * Hk * Q * D * e);
  L->nv = take(B * Hk * Q * Dv * e);
  L->ctx = take(B * Hq * Q * Dv * e);
  L->bytes = off;
  (void)M;
  return true;
}

// ---- scratch for the no-allocation step ----
// A file-scope device array that serves as the step's workspace for callers
// that cannot allocate (kvc_step_inplace_noalloc).  Every GPU the library
// runs on holds its own copy until the process ends.  Host code never uses
// the array's name as an address: scratch_address() looks up each device's
// copy once, with that device current, and keeps it.
constexpr size_t kScratchBytes = size_t(96) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// The device `stream` runs on (the current device for the null stream).
int stream_device(hipStream_t stream, int* dev) {
  if (stream) return hipStreamGetDevice(stream, dev) == hipSuccess ? KVC_OK : KVC_ERR_HIP;
  return hipGetDevice(dev) == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// Address of device `dev`'s copy of `scratch`, looked up on first use.
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return KVC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return KVC_ERR_HIP;
    if (prev != dev && hipSetDevice(dev) != hipSuccess) return KVC_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return KVC_ERR_HIP;
    }
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return KVC_OK;
}

}  // namespace

extern "C" {

size_t kvc_noalloc_scratch_bytes(void) { return kScratchBytes; }

int kvc_step_inplace_noalloc(const kvc_dims* dims, int dtype, int has_scale, double scale,
                             const void* query, const void* new_key, const void* new_value,
                             void* key_cache, void* value_cache, const int64_t* lengths,
                             const uint8_t* append_mask, int64_t* lengths_out, void* attention,
                             void* context, int32_t* row_status, void* stream,
                             const kvc_events* events) {
  Plan p;
  int rc = make_plan(dims, dtype, &p);
  if (rc != KVC_OK) return rc;
  if (p.pub.workspace_bytes > kScratchBytes) return KVC_ERR_TOO_LARGE;
  int dev = 0;
  rc = stream_device(static_cast<hipStream_t>(stream), &dev);
  if (rc != KVC_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(dev, &ws);
  if (rc != KVC_OK) return rc;
  return run_step(dims, dtype, has_scale, scale, query, new_key, new_value, key_cache,
                  value_cache, key_cache, value_cache, false, lengths, append_mask, lengths_out,
                  attention, context, row_status, ws, kScratchBytes, stream, events);
}

size_t kvc_attend_workspace_bytes(const kvc_dims* dims, int dtype) {
  ReattLayout L;
  return dims && reatt_layout(dims, dtype, &L) ? L.bytes : 0;
}

int kvc_attend_over_cache(const kvc_dims* dims, int dtype, int has_scale, double scale,
                          const void* q, int64_t total_q, const int64_t* cu_seqlens_q,
                          const void* key_cache, const void* value_cache, int64_t num_blocks,
                          int64_t block_size, const int32_t* block_table, const int32_t* slot_ids,
                          const int64_t* seqlens_k, int64_t seqlens_k_count,
                          const float* head_sink, void* out,
                          int32_t* row_status, void* workspace, size_t workspace_bytes,
                          void* stream, const kvc_events* events) {
  if (!dims) return KVC_ERR_NULL;
  const kvc_dims* d = dims;
  int rc = check_dims(d, dtype);
  if (rc != KVC_OK) return rc;
  double sc;
  rc = check_scale(has_scale, scale, d->D, &sc);
  if (rc != KVC_OK) return rc;
  ReattLayout L;
  if (!reatt_layout(d, dtype, &L)) return KVC_ERR_SHAPE;
  if (total_q < 0 || num_blocks < 1) return KVC_ERR_SHAPE;
  if (seqlens_k_count != d->B && seqlens_k_count != d->B + 1) return KVC_ERR_SHAPE;
  if (!cu_seqlens_q || !key_cache || !value_cache || !seqlens_k || !workspace) return KVC_ERR_NULL;
  if (total_q > 0 && (!q || !out)) return KVC_ERR_NULL;
  if (workspace_bytes < L.bytes) return KVC_ERR_WORKSPACE;
  int64_t x;
  if (!mul_ok(total_q, d->Hq, kMaxElems, &x) || !mul_ok(x, d->D > d->Dv ? d->D : d->Dv, kMaxElems, &x))
    return KVC_ERR_SHAPE;

  // the cache: a block pool with a table, a continuous cache whose rows
  // slot_ids picks (one block of M rows per sequence), or the continuous
  // cache read row b for sequence b
  PagedPool pg{num_blocks, block_size, nullptr, false};
  const PagedPool* pgp = nullptr;
  if (block_table) {
    if (slot_ids) return KVC_ERR_SHAPE;  // one layout at a time
    pg.table = block_table;
    pgp = &pg;
  } else {
    if (block_size != d->M && block_size != 0) return KVC_ERR_SHAPE;
    pg.block_size = d->M;
    if (slot_ids) {
      pg.table = slot_ids;
      pgp = &pg;
    } else if (num_blocks < d->B) {
      return KVC_ERR_SHAPE;
    }
  }
  if (pgp) {  // the check the step makes on the mapped cache, before anything is enqueued
    const int64_t bs = pg.block_size;
    const bool single = bs == d->M;
    if (bs < 1 || (!single && ((bs & (bs - 1)) != 0 || d->M % bs != 0))) return KVC_ERR_SHAPE;
  }
  const size_t e = dtype == KVC_F32 ? 4 : 2;
  const size_t B = d->B, Hq = d->Hq, Hk = d->Hk, Tq = total_q, D = d->D, Dv = d->Dv;
  const size_t rows = static_cast<size_t>(num_blocks) * static_cast<size_t>(pg.block_size);
  const size_t tab = block_table ? B * static_cast<size_t>(d->M / pg.block_size) * 4
                                 : (slot_ids ? B * 4 : 0);
  const Range r_q{q, Tq * Hq * D * e}, r_cu{cu_seqlens_q, (B + 1) * 8},
      r_kc{key_cache, rows * Hk * D * e}, r_vc{value_cache, rows * Hk * Dv * e},
      r_tab{block_table ? static_cast<const void*>(block_table) : slot_ids, tab},
      r_lk{seqlens_k, static_cast<size_t>(seqlens_k_count) * 8},
      r_sink{head_sink, head_sink ? Hq * 4 : 0},
      r_out{out, Tq * Hq * Dv * e}, r_st{row_status, row_status ? B * 4 : 0},
      r_ws{workspace, L.bytes};
  const Range ins[] = {r_q, r_cu, r_kc, r_vc, r_tab, r_lk, r_sink};
  const Range outs[] = {r_out, r_st, r_ws};
  for (int i = 0; i < 3; i++) {
    for (const Range& in : ins)
      if (overlap(outs[i], in)) return KVC_ERR_ALIAS;
    for (int j = i + 1; j < 3; j++)
      if (overlap(outs[i], outs[j])) return KVC_ERR_ALIAS;
  }

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  (void)hipGetLastError();  // an earlier error is not ours
  StepArgs a;
  std::memset(&a, 0, sizeof a);
  a.B = d->B; a.Hq = d->Hq; a.Hk = d->Hk; a.Q = d->Q; a.M = d->M; a.D = d->D; a.Dv = d->Dv;
  a.G = static_cast<int32_t>(d->Hq / d->Hk);
  a.elem_bytes = static_cast<int64_t>(e);
  a.kc_in = key_cache;
  a.vc_in = value_cache;
  if (pgp) set_paged(a, d, *pgp);
  kvc::ReattArgs r;
  r.Tq = total_q;
  r.q = static_cast<const uint8_t*>(q);
  r.cu_q = cu_seqlens_q;
  r.seqlens_k = seqlens_k;
  r.cum_k = seqlens_k_count == d->B + 1 ? 1 : 0;
  r.out = static_cast<uint8_t*>(out);
  r.row_status = row_status;
  r.len0 = reinterpret_cast<int64_t*>(ws + L.len0);
  r.mask = ws + L.mask;
  r.qs = ws + L.qs;
  r.nk = ws + L.nk;
  r.nv = ws + L.nv;
  r.rstat = reinterpret_cast<int32_t*>(ws + L.rstat);
  r.ctx = ws + L.ctx;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(kvc::reattend_prep_kernel, dim3(static_cast<unsigned>(d->B)),
                     dim3(kvc::kReattThreads), 0, s, a, r);
  rc = run_step(d, dtype, has_scale, scale, r.qs, r.nk, r.nv, key_cache, value_cache,
                const_cast<void*>(key_cache), const_cast<void*>(value_cache), false, r.len0,
                r.mask, reinterpret_cast<int64_t*>(ws + L.lens_out), nullptr, ws + L.ctx,
                reinterpret_cast<int32_t*>(ws + L.status), workspace, L.step, stream, events,
                pgp, true, head_sink);
  if (rc != KVC_OK) return rc;
  hipLaunchKernelGGL(kvc::reattend_scatter_kernel, dim3(static_cast<unsigned>(d->B)),
                     dim3(kvc::kReattThreads), 0, s, a, r);
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

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

int kvc_step_paged(const kvc_dims* dims, int dtype, int has_scale, double scale,
                   const void* query, const void* new_key, const void* new_value, void* key_pool,
                   void* value_pool, int64_t num_blocks, int64_t block_size,
                   const int32_t* block_table, const int64_t* lengths, const uint8_t* append_mask,
                   int64_t* lengths_out, void* attention, void* context, int32_t* row_status,
                   void* workspace, size_t workspace_bytes, void* stream,
                   const kvc_events* events) {
  const PagedPool pg{num_blocks, block_size, block_table, false};
  return run_step(dims, dtype, has_scale, scale, query, new_key, new_value, key_pool, value_pool,
                  key_pool, value_pool, false, lengths, append_mask, lengths_out, attention,
                  context, row_status, workspace, workspace_bytes, stream, events, &pg);
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
    case KVC_ERR_TOO_LARGE: return "the step needs more workspace than the no-allocation entry "
                                   "point's static scratch holds";
    case KVC_ERR_UNSUPPORTED: return "a shape, block size or buffer alignment the entry point "
                                     "does not take";
    case KVC_ROW_BAD_LENGTH: return "row rejected: length outside [0, M]";
    case KVC_ROW_OVERFLOW: return "row rejected: length + n exceeds M";
    case KVC_ROW_NOT_PREFIX: return "row rejected: append mask is not a prefix";
    case KVC_ROW_BAD_QUERIES: return "sequence rejected: query range outside the packed queries, "
                                     "longer than Q or than the cached length";
    default: return "unknown code";
  }
}

}  // extern "C"
