// Host-side argument validation and status strings of libsattn.
//
// The shape rule is the admission predicate of the StreamingAttentionSM86
// page (the forward's admission definition): T, Hq and Hkv nonzero, Hq a
// multiple of Hkv, Hq <= 65535 and Hq * 64 * T * 4 <= 2^32 - 1 (the
// largest plane then fits 32-bit byte offsets).  The page also requires T to
// be a multiple of 64; this library drops that condition and masks the last,
// partial tile instead.  c > 0 follows from the page masking scores before
// scaling them, which keeps -inf only for a positive scale.
//
// This file makes no HIP call, so it builds with a plain host compiler too.
#include <math.h>
#include <stdint.h>

#include "sattn.h"

namespace {

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

Span span(const void* p, uint64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{lo, lo + static_cast<uintptr_t>(bytes)};
}

}  // namespace

extern "C" int sattn_fwd_check(const void* Q, const void* K, const void* Vt, const void* O,
                               const float* L, float c, int T, int Hq, int Hkv) {
  if (!Q || !K || !Vt || !O || !L) return SATTN_ERR_NULL;
  if (T < 1 || Hq < 1 || Hkv < 1) return SATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq > 65535) return SATTN_ERR_SHAPE;
  const uint64_t t = static_cast<uint64_t>(T);
  const uint64_t hq = static_cast<uint64_t>(Hq);
  const uint64_t hkv = static_cast<uint64_t>(Hkv);
  if (hq * SATTN_HEAD_DIM * t * 4u > 0xFFFFFFFFull) return SATTN_ERR_SHAPE;
  if (!isfinite(c) || !(c > 0.0f)) return SATTN_ERR_SCALE;
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) |
                        reinterpret_cast<uintptr_t>(Vt) | reinterpret_cast<uintptr_t>(O);
  if ((a16 & 15u) != 0 || (reinterpret_cast<uintptr_t>(L) & 3u) != 0) return SATTN_ERR_ALIGN;
  const uint64_t plane = t * SATTN_HEAD_DIM * 2u;  // bytes of one [T][64] binary16 head
  const Span q = span(Q, hq * plane), k = span(K, hkv * plane), v = span(Vt, hkv * plane);
  const Span o = span(O, hq * plane), l = span(L, hq * t * 4u);
  if (overlaps(o, q) || overlaps(o, k) || overlaps(o, v) || overlaps(o, l)) return SATTN_ERR_ALIAS;
  if (overlaps(l, q) || overlaps(l, k) || overlaps(l, v)) return SATTN_ERR_ALIAS;
  return SATTN_OK;
}

extern "C" const char* sattn_status_string(int status) {
  switch (status) {
    case SATTN_OK: return "ok";
    case SATTN_ERR_NULL: return "a required pointer is NULL";
    case SATTN_ERR_SHAPE:
      return "bad shape: need T >= 1, Hq >= 1, Hkv >= 1, Hq % Hkv == 0, Hq <= 65535 and "
             "Hq*64*T*4 <= 2^32-1";
    case SATTN_ERR_SCALE: return "the scale c must be finite and > 0";
    case SATTN_ERR_ALIGN: return "Q, K, Vt and O must be 16-byte aligned and L 4-byte aligned";
    case SATTN_ERR_ALIAS: return "O or L overlaps an input or each other";
    case SATTN_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
    case SATTN_ERR_LAUNCH: return "the kernel launch failed";
    default: return "unknown sattn status";
  }
}
