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
#include "sattn_check.h"

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

namespace {

int check_shape_scale(float c, int T, int Hq, int Hkv) {
  if (T < 1 || Hq < 1 || Hkv < 1) return SATTN_ERR_SHAPE;
  if (Hq % Hkv != 0 || Hq > 65535) return SATTN_ERR_SHAPE;
  if (static_cast<uint64_t>(Hq) * SATTN_HEAD_DIM * static_cast<uint64_t>(T) * 4u > 0xFFFFFFFFull)
    return SATTN_ERR_SHAPE;
  if (!isfinite(c) || !(c > 0.0f)) return SATTN_ERR_SCALE;
  return SATTN_OK;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// The argument set of one backward launch; absent pointers are NULL and
// `need` says which of them the launch requires.
struct BwdArgs {
  const void *Q, *K, *Vt, *O, *dO, *L;      // inputs
  const void *dQ, *D_out, *dK, *dVt, *ws;   // outputs (D is an input of the key launch)
  const void* D_in;
  unsigned long long wsBytes;
  float c, s;
  int T, Hq, Hkv;
  // nonzero: the workspace is the library's own static region of this many
  // bytes (ws is ignored; it cannot overlap caller buffers)
  unsigned long long libWsBytes = 0;
};

int check_bwd(const BwdArgs& a, bool query, bool key) {
  if (!a.Q || !a.K || !a.Vt || !a.dO || !a.L) return SATTN_ERR_NULL;
  if (query && (!a.O || !a.dQ || !a.D_out)) return SATTN_ERR_NULL;
  if (key && (!a.dK || !a.dVt)) return SATTN_ERR_NULL;
  if (key && !query && !a.D_in) return SATTN_ERR_NULL;
  int st = check_shape_scale(a.c, a.T, a.Hq, a.Hkv);
  if (st != SATTN_OK) return st;
  if (!isfinite(a.s) || !(a.s > 0.0f)) return SATTN_ERR_SCALE;
  const unsigned long long need = sattn_bwd_workspace_bytes(a.T, a.Hq, a.Hkv);
  if (key && need > 0 && a.libWsBytes > 0 && need > a.libWsBytes) return SATTN_ERR_SCRATCH;
  if (key && need > 0 && a.libWsBytes == 0 && (!a.ws || a.wsBytes < need))
    return SATTN_ERR_WORKSPACE;
  if (misaligned(a.Q, 16) || misaligned(a.K, 16) || misaligned(a.Vt, 16) ||
      misaligned(a.dO, 16) || misaligned(a.L, 4))
    return SATTN_ERR_ALIGN;
  if (query && (misaligned(a.O, 16) || misaligned(a.dQ, 16) || misaligned(a.D_out, 4)))
    return SATTN_ERR_ALIGN;
  if (key && (misaligned(a.dK, 16) || misaligned(a.dVt, 16) ||
              (a.libWsBytes == 0 && misaligned(a.ws, 16)) || misaligned(a.D_in, 4)))
    return SATTN_ERR_ALIGN;
  const uint64_t t = static_cast<uint64_t>(a.T);
  const uint64_t hq = static_cast<uint64_t>(a.Hq), hkv = static_cast<uint64_t>(a.Hkv);
  const uint64_t half = t * SATTN_HEAD_DIM * 2u, word = t * SATTN_HEAD_DIM * 4u;
  Span in[7];
  int nIn = 0;
  in[nIn++] = span(a.Q, hq * half);
  in[nIn++] = span(a.K, hkv * half);
  in[nIn++] = span(a.Vt, hkv * half);
  in[nIn++] = span(a.dO, hq * half);
  in[nIn++] = span(a.L, hq * t * 4u);
  if (query) in[nIn++] = span(a.O, hq * half);
  if (key && !query) in[nIn++] = span(a.D_in, hq * t * 4u);
  Span out[5];
  int nOut = 0;
  if (query) {
    out[nOut++] = span(a.dQ, hq * word);
    out[nOut++] = span(a.D_out, hq * t * 4u);
  }
  if (key) {
    out[nOut++] = span(a.dK, hkv * word);
    out[nOut++] = span(a.dVt, hkv * word);
    if (need > 0 && a.libWsBytes == 0) out[nOut++] = span(a.ws, need);
  }
  for (int i = 0; i < nOut; ++i) {
    for (int j = 0; j < nIn; ++j)
      if (overlaps(out[i], in[j])) return SATTN_ERR_ALIAS;
    for (int j = i + 1; j < nOut; ++j)
      if (overlaps(out[i], out[j])) return SATTN_ERR_ALIAS;
  }
  return SATTN_OK;
}

}  // namespace

extern "C" unsigned long long sattn_bwd_workspace_bytes(int T, int Hq, int Hkv) {
  if (check_shape_scale(1.0f, T, Hq, Hkv) != SATTN_OK || Hq == Hkv) return 0;
  return 2ull * static_cast<unsigned long long>(Hq) * static_cast<unsigned long long>(T) *
         SATTN_HEAD_DIM * 4ull;
}

extern "C" int sattn_bwd_check(const void* Q, const void* K, const void* Vt, const void* O,
                               const void* dO, const float* L, const float* dQ, const float* dK,
                               const float* dVt, const float* D, const void* workspace,
                               unsigned long long workspace_bytes, float c, float s, int T,
                               int Hq, int Hkv) {
  const BwdArgs a{Q, K, Vt, O, dO, L, dQ, D, dK, dVt, workspace, nullptr, workspace_bytes,
                  c, s, T, Hq, Hkv};
  return check_bwd(a, true, true);
}

extern "C" int sattn_bwd_query_check(const void* Q, const void* K, const void* Vt, const void* O,
                                     const void* dO, const float* L, const float* dQ,
                                     const float* D, float c, float s, int T, int Hq, int Hkv) {
  const BwdArgs a{Q, K, Vt, O, dO, L, dQ, D, nullptr, nullptr, nullptr, nullptr, 0,
                  c, s, T, Hq, Hkv};
  return check_bwd(a, true, false);
}

extern "C" int sattn_bwd_key_check(const void* Q, const void* K, const void* Vt, const void* dO,
                                   const float* L, const float* D, const float* dK,
                                   const float* dVt, const void* workspace,
                                   unsigned long long workspace_bytes, float c, float s, int T,
                                   int Hq, int Hkv) {
  const BwdArgs a{Q, K, Vt, nullptr, dO, L, nullptr, nullptr, dK, dVt, workspace, D,
                  workspace_bytes, c, s, T, Hq, Hkv};
  return check_bwd(a, false, true);
}

// The validation of sattn_bwd_key_noalloc: as sattn_bwd_key_check, with the
// workspace replaced by the library's static region of `scratch_bytes`.
int sattn_bwd_key_noalloc_check(const void* Q, const void* K, const void* Vt, const void* dO,
                                const float* L, const float* D, const float* dK,
                                const float* dVt, float c, float s, int T, int Hq, int Hkv,
                                unsigned long long scratch_bytes) {
  BwdArgs a{Q, K, Vt, nullptr, dO, L, nullptr, nullptr, dK, dVt, nullptr, D, 0,
            c, s, T, Hq, Hkv};
  a.libWsBytes = scratch_bytes;
  return check_bwd(a, false, true);
}

extern "C" int sattn_mat_fwd_check(const void* Q, const void* K, const void* Vt, const void* O,
                                   const float* L, const float* S, const void* P, float c, int T,
                                   int Hq, int Hkv) {
  if (!Q || !K || !Vt || !O || !L || !S || !P) return SATTN_ERR_NULL;
  const int st = check_shape_scale(c, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const uint64_t t = static_cast<uint64_t>(T);
  const uint64_t hq = static_cast<uint64_t>(Hq), hkv = static_cast<uint64_t>(Hkv);
  const uint64_t plane = hq * t * t;  // elements of S and of P
  if (plane * 4u > (1ull << 40)) return SATTN_ERR_SHAPE;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(Vt, 16) || misaligned(O, 16) ||
      misaligned(S, 16) || misaligned(P, 16) || misaligned(L, 4))
    return SATTN_ERR_ALIGN;
  const uint64_t half = t * SATTN_HEAD_DIM * 2u;
  const Span in[3] = {span(Q, hq * half), span(K, hkv * half), span(Vt, hkv * half)};
  const Span out[4] = {span(O, hq * half), span(L, hq * t * 4u), span(S, plane * 4u),
                       span(P, plane * 2u)};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlaps(out[i], in[j])) return SATTN_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out[j])) return SATTN_ERR_ALIAS;
  }
  return SATTN_OK;
}

namespace {

int mat_shape(int T, int Hq, int Hkv) {
  const int st = check_shape_scale(1.0f, T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  const uint64_t t = static_cast<uint64_t>(T);
  if (static_cast<uint64_t>(Hq) * t * t * 4u > (1ull << 40)) return SATTN_ERR_SHAPE;
  return SATTN_OK;
}

int disjoint(const Span* in, int nIn, const Span* out, int nOut) {
  for (int i = 0; i < nOut; ++i) {
    for (int j = 0; j < nIn; ++j)
      if (overlaps(out[i], in[j])) return SATTN_ERR_ALIAS;
    for (int j = i + 1; j < nOut; ++j)
      if (overlaps(out[i], out[j])) return SATTN_ERR_ALIAS;
  }
  return SATTN_OK;
}

}  // namespace

extern "C" int sattn_mat_scores_check(const void* Q, const void* K, const float* S, float c,
                                      int T, int Hq, int Hkv) {
  if (!Q || !K || !S) return SATTN_ERR_NULL;
  int st = mat_shape(T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  if (!isfinite(c) || !(c > 0.0f)) return SATTN_ERR_SCALE;
  if (misaligned(Q, 16) || misaligned(K, 16) || misaligned(S, 16)) return SATTN_ERR_ALIGN;
  const uint64_t t = static_cast<uint64_t>(T), half = t * SATTN_HEAD_DIM * 2u;
  const Span in[2] = {span(Q, static_cast<uint64_t>(Hq) * half),
                      span(K, static_cast<uint64_t>(Hkv) * half)};
  const Span out[1] = {span(S, static_cast<uint64_t>(Hq) * t * t * 4u)};
  return disjoint(in, 2, out, 1);
}

extern "C" int sattn_mat_softmax_check(const float* S, const void* P, const float* L, int T,
                                       int Hq) {
  if (!S || !P || !L) return SATTN_ERR_NULL;
  int st = mat_shape(T, Hq, 1);
  if (st != SATTN_OK) return st;
  if (misaligned(S, 16) || misaligned(P, 16) || misaligned(L, 4)) return SATTN_ERR_ALIGN;
  const uint64_t t = static_cast<uint64_t>(T), plane = static_cast<uint64_t>(Hq) * t * t;
  const Span in[1] = {span(S, plane * 4u)};
  const Span out[2] = {span(P, plane * 2u), span(L, static_cast<uint64_t>(Hq) * t * 4u)};
  return disjoint(in, 1, out, 2);
}

extern "C" int sattn_mat_pv_check(const void* P, const void* Vt, const void* O, int T, int Hq,
                                  int Hkv) {
  if (!P || !Vt || !O) return SATTN_ERR_NULL;
  int st = mat_shape(T, Hq, Hkv);
  if (st != SATTN_OK) return st;
  if (misaligned(P, 16) || misaligned(Vt, 16) || misaligned(O, 16)) return SATTN_ERR_ALIGN;
  const uint64_t t = static_cast<uint64_t>(T), half = t * SATTN_HEAD_DIM * 2u;
  const Span in[2] = {span(P, static_cast<uint64_t>(Hq) * t * t * 2u),
                      span(Vt, static_cast<uint64_t>(Hkv) * half)};
  const Span out[1] = {span(O, static_cast<uint64_t>(Hq) * half)};
  return disjoint(in, 2, out, 1);
}

extern "C" const char* sattn_status_string(int status) {
  switch (status) {
    case SATTN_OK: return "ok";
    case SATTN_ERR_NULL: return "a required pointer is NULL";
    case SATTN_ERR_SHAPE:
      return "bad shape: need T >= 1, Hq >= 1, Hkv >= 1, Hq % Hkv == 0, Hq <= 65535 and "
             "Hq*64*T*4 <= 2^32-1";
    case SATTN_ERR_SCALE: return "the scales c and s must be finite and > 0";
    case SATTN_ERR_ALIGN:
      return "binary16 arrays, dQ, dK, dVt and the workspace must be 16-byte aligned, L and D "
             "4-byte aligned";
    case SATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case SATTN_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
    case SATTN_ERR_LAUNCH: return "the kernel launch failed";
    case SATTN_ERR_WORKSPACE: return "the workspace is NULL or smaller than sattn_bwd_workspace_bytes()";
    case SATTN_ERR_SCRATCH:
      return "the problem needs more workspace than sattn_bwd_key_noalloc's static region "
             "(SATTN_BWD_NOALLOC_MAX_BYTES)";
    default: return "unknown sattn status";
  }
}
