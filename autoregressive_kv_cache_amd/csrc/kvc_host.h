// kvc_host.h -- host-side checks shared by the library's entry points:
// shape limits, the softmax scale, buffer overlap and layout arithmetic.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/kvc.h"

namespace kvc_host {

constexpr int64_t kMaxElems = int64_t(1) << 46;    // per tensor

// a * b with an overflow / limit check
inline bool mul_ok(int64_t a, int64_t b, int64_t limit, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > limit / a) return false;
  *out = a * b;
  return *out <= limit;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int check_dims(const kvc_dims* d, int dtype) {
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

inline int check_scale(int has_scale, double scale, int64_t D, double* out) {
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

inline bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

}  // namespace kvc_host
