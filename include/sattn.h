/*
 * libsattn: the causal streaming-attention forward on AMD MI355X (gfx950).
 *
 * What is computed (StreamingAttentionSM86 page, header comment of the forward
 * realization): for every query head h and query row i,
 *
 *     t_ij = c * (q_i . k_j)                      for keys j <= i (diagonal kept)
 *     O[i][h*64 + d] = sum_j 2^t_ij * V_j[d] / sum_j 2^t_ij
 *     L[h][i]        = log2 sum_j 2^t_ij          (base-2 log-sum-exp)
 *
 * folded tile by tile with a running row maximum m, row sum l and weighted
 * sum, so the T x T scores never exist in memory.  The probabilities
 * P = 2^(t - m) are rounded to binary16 (round to nearest even) before their
 * product with V; every sum stays binary32.  Query head h reads K/V head
 * h / G with G = Hq / Hkv (the page numbers query heads kvHead * G + z).
 *
 * The constant c is the binary32 nearest scale / ln 2; with scale = 1/sqrt(64)
 * it is 0x3E38AA3B (Graph page, cgStreamingScale).
 *
 * All functions are thread-safe.  No entry point allocates memory or keeps
 * state between calls besides a per-device cache of the architecture check.
 */
#ifndef SATTN_H
#define SATTN_H

#ifdef __cplusplus
extern "C" {
#endif

#define SATTN_HEAD_DIM 64

typedef enum {
  SATTN_OK = 0,
  SATTN_ERR_NULL = 1,   /* Q, K, Vt, O or L is NULL                                  */
  SATTN_ERR_SHAPE = 2,  /* T < 1, Hq < 1, Hkv < 1, Hq % Hkv != 0, Hq > 65535, or
                           Hq * 64 * T * 4 > 2^32 - 1                                 */
  SATTN_ERR_SCALE = 3,  /* c is not finite or c <= 0                                  */
  SATTN_ERR_ALIGN = 4,  /* Q, K, Vt or O not 16-byte aligned, or L not 4-byte aligned */
  SATTN_ERR_ALIAS = 5,  /* O or L overlaps Q, K, Vt, or each other                    */
  SATTN_ERR_DEVICE = 6, /* no current HIP device, or it is not gfx950                 */
  SATTN_ERR_LAUNCH = 7  /* the kernel launch was refused (hipGetLastError)            */
} sattn_status;

/*
 * sattn_fwd: enqueue the causal streaming-attention forward on `stream`.
 * Defined by the StreamingAttentionSM86 page (forward realization, its header
 * comment, its tile body and its epilogue); argument order follows that
 * kernel's parameter list: Q, K, V^T, O, L, then c.
 *
 *   Q    device, binary16 [Hq][T][64], row-major (query head, token, width)
 *   K    device, binary16 [Hkv][T][64]
 *   Vt   device, binary16 [Hkv][64][T]  (V transposed per head)
 *   O    device, binary16 [T][Hq*64], token-major with the heads merged:
 *        element (i, h, d) at i*Hq*64 + h*64 + d; every element is written
 *   L    device, binary32 [Hq][T]: element (h, i) at h*T + i, base-2 units;
 *        every element is written
 *   c    binary32 base-2 score scale, finite and > 0
 *   T    tokens (any value >= 1; it need not be a multiple of 64)
 *   Hq   query heads, Hkv K/V heads, Hq a multiple of Hkv
 *   stream  a hipStream_t, or NULL for the default stream
 *
 * Ownership: every buffer belongs to the caller; nothing is retained after
 * the call returns.  Q, K and Vt may overlap one another (they are only read);
 * O and L must not overlap anything.
 *
 * Errors: arguments are validated (as sattn_fwd_check does) before anything
 * is enqueued; on any error nothing is launched and O and L are untouched.
 * The call is asynchronous: it returns once the kernel is enqueued, and a
 * fault during execution surfaces at the caller's next synchronisation.
 * Results are deterministic: the same inputs give the same bits on every run.
 */
int sattn_fwd(const void* Q, const void* K, const void* Vt, void* O, float* L,
              float c, int T, int Hq, int Hkv, void* stream);

/*
 * sattn_fwd_check: the host-side argument validation of sattn_fwd alone
 * (the admission rule of the StreamingAttentionSM86 page, with T no longer
 * required to be a multiple of 64, plus pointer checks).  Makes no HIP call,
 * dereferences no pointer and launches nothing; returns the status sattn_fwd
 * would return before touching the device (never SATTN_ERR_DEVICE or
 * SATTN_ERR_LAUNCH).
 */
int sattn_fwd_check(const void* Q, const void* K, const void* Vt, const void* O,
                    const float* L, float c, int T, int Hq, int Hkv);

/* sattn_status_string: a static, NUL-terminated description of a status code
 * (an unknown code gives "unknown sattn status").  Never NULL. */
const char* sattn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SATTN_H */
