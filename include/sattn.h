/*
 * libsattn: causal streaming attention, forward and backward, on AMD MI355X
 * (gfx950).
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
 * state between calls besides a per-device cache of the architecture check
 * (and, for sattn_bwd_key_noalloc, of its static region's address).
 */
#ifndef SATTN_H
#define SATTN_H

#ifdef __cplusplus
extern "C" {
#endif

#define SATTN_HEAD_DIM 64

typedef enum {
  SATTN_OK = 0,
  SATTN_ERR_NULL = 1,   /* a required pointer is NULL                               */
  SATTN_ERR_SHAPE = 2,  /* T < 1, Hq < 1, Hkv < 1, Hq % Hkv != 0, Hq > 65535, or
                           Hq * 64 * T * 4 > 2^32 - 1                                 */
  SATTN_ERR_SCALE = 3,  /* c (or the backward's s) is not finite, or is <= 0         */
  SATTN_ERR_ALIGN = 4,  /* a pointer is less aligned than its entry point requires    */
  SATTN_ERR_ALIAS = 5,  /* an output overlaps an input or another output              */
  SATTN_ERR_DEVICE = 6, /* no current HIP device, or it is not gfx950                 */
  SATTN_ERR_LAUNCH = 7, /* the kernel launch was refused (hipGetLastError)            */
  SATTN_ERR_WORKSPACE = 8, /* the backward's workspace is NULL or smaller than needed  */
  SATTN_ERR_SCRATCH = 9    /* sattn_bwd_key_noalloc: the problem needs more workspace
                              than its static region holds                            */
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
 * sattn_fwd_vrows: sattn_fwd with V given as rows, binary16 [Hkv][T][64]
 * (V of K/V head kv, token j at (kv*T + j)*64), the layout the value
 * projection produces, instead of V^T; everything else, the results
 * included, is as for sattn_fwd (bit-identical O and L for the same values).
 * It removes the value-transpose step before the attention (the Graph page's
 * cgLayerForwardWith launches the value-transpose image on the layer's QKV
 * plane before the attention; the DeviceImages page lists that image in
 * coppeliusCoreDeviceImages): the kernel reads the V^T operand of P V from
 * row-major V tiles with the gfx950 LDS transpose read.  V must be 16-byte
 * aligned; validation as sattn_fwd.
 */
int sattn_fwd_vrows(const void* Q, const void* K, const void* V, void* O, float* L, float c,
                    int T, int Hq, int Hkv, void* stream);

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

/*
 * The backward (StreamingAttentionSM86 page: the comment that opens the
 * backward pass and those of its query launch, key launch and grouped
 * gradient reduction).  With the forward's O and L and the output gradient
 * dO, and P_ij = 2^(c (q_i . k_j) - L_i) for keys j <= i (else 0):
 *
 *     D_i   = sum_d dO_id O_id            (the row term)
 *     dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = s sum_j dS_ij k_j
 *     dK_j  = s sum_i dS_ij q_i,   dV_j = sum_i P_ij dO_i
 *
 * where the key gradients of a K/V head are summed over the G query heads of
 * its group.  P and dS are rounded to binary16 (round to nearest even) as the
 * operands of the products that follow; every sum is binary32.  With
 * c = s log2(e) and the forward's own O and L these are the gradients of
 * sum(dO * O) with respect to Q, K and V.  Deterministic: no atomics, and
 * every sum, the group sum included, is taken in an order fixed by T and Hq,
 * so the same inputs give the same bits on every run.
 *
 * Shared arguments (layouts as in sattn_fwd):
 *   Q    device, binary16 [Hq][T][64];  K  device, binary16 [Hkv][T][64]
 *   Vt   device, binary16 [Hkv][64][T]
 *   O    device, binary16 [T][Hq*64], the forward's output (token-major)
 *   dO   device, binary16 [T][Hq*64], the output gradient, laid out like O
 *   L    device, binary32 [Hq][T], the forward's base-2 log-sum-exp
 *   c    binary32 base-2 score scale (finite, > 0), as given to sattn_fwd
 *   s    binary32 natural score scale (finite, > 0) applied to dQ and dK
 *   T, Hq, Hkv as in sattn_fwd; stream a hipStream_t or NULL
 * Buffers are the caller's and nothing is retained; inputs may overlap one
 * another, outputs may overlap nothing.  Pointers to binary16 data must be
 * 16-byte aligned, to binary32 data 16-byte aligned (L: 4-byte).  Arguments
 * are validated before anything is enqueued (on error nothing is launched and
 * no output is touched); calls are asynchronous like sattn_fwd.
 */

/*
 * sattn_bwd_query: the query launch.  Writes the row term D (binary32
 * [Hq][T], every element) and dQ (binary32 [Hq][T][64], row-major per query
 * head, every element).
 */
int sattn_bwd_query(const void* Q, const void* K, const void* Vt, const void* O,
                    const void* dO, const float* L, float* dQ, float* D, float c, float s,
                    int T, int Hq, int Hkv, void* stream);

/*
 * sattn_bwd_key: the key launch and, when Hq > Hkv, the grouped gradient
 * reduction.  Reads D as written by sattn_bwd_query (enqueue that first on the
 * same stream).  Writes dK (binary32 [Hkv][T][64]) and the V gradient
 * transposed like V^T, dVt (binary32 [Hkv][64][T]); every element of both.
 *
 *   workspace        device scratch of at least sattn_bwd_workspace_bytes()
 *                    bytes, 16-byte aligned, holding one dK and one dV^T
 *                    plane per query head between the two launches; may be
 *                    NULL when that size is 0.  Its contents on entry do not
 *                    matter; on return they are unspecified.  Calls that share
 *                    a workspace must be ordered (one stream).
 *   workspace_bytes  its size; SATTN_ERR_WORKSPACE if too small.
 */
int sattn_bwd_key(const void* Q, const void* K, const void* Vt, const void* dO,
                  const float* L, const float* D, float* dK, float* dVt, void* workspace,
                  unsigned long long workspace_bytes, float c, float s, int T, int Hq, int Hkv,
                  void* stream);

/*
 * sattn_bwd_key_noalloc: sattn_bwd_key for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the per-query-head planes that sattn_bwd_key keeps
 * in the caller's workspace live instead in one static device region of the
 * library, SATTN_BWD_NOALLOC_MAX_BYTES (64 MiB) on each GPU the library runs
 * on, held until the process ends.  No call allocates or frees anything.
 * Arguments, layouts, results (bit-identical to sattn_bwd_key's) and
 * validation as sattn_bwd_key without the workspace; SATTN_ERR_SCRATCH when
 * sattn_bwd_workspace_bytes(T, Hq, Hkv) exceeds SATTN_BWD_NOALLOC_MAX_BYTES
 * (nothing is launched).  Every call on a GPU uses that GPU's one region:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it and give wrong dK and dVt, so such calls must be ordered (one
 * stream, or events).  The region's contents on entry do not matter.
 */
#define SATTN_BWD_NOALLOC_MAX_BYTES (64ull << 20)
int sattn_bwd_key_noalloc(const void* Q, const void* K, const void* Vt, const void* dO,
                          const float* L, const float* D, float* dK, float* dVt, float c,
                          float s, int T, int Hq, int Hkv, void* stream);

/*
 * sattn_bwd: sattn_bwd_query then sattn_bwd_key on `stream`; the outputs of
 * both (D is an output too).
 */
int sattn_bwd(const void* Q, const void* K, const void* Vt, const void* O, const void* dO,
              const float* L, float* dQ, float* dK, float* dVt, float* D, void* workspace,
              unsigned long long workspace_bytes, float c, float s, int T, int Hq, int Hkv,
              void* stream);

/* sattn_bwd_workspace_bytes: the workspace sattn_bwd_key and sattn_bwd need:
 * 0 when Hq == Hkv, else 2 * Hq * T * 64 * 4 bytes; 0 for shapes that
 * sattn_bwd_check rejects.  Makes no HIP call. */
unsigned long long sattn_bwd_workspace_bytes(int T, int Hq, int Hkv);

/*
 * sattn_bwd_check: the host-side validation of sattn_bwd alone (shape rule
 * and scales as for sattn_fwd, s finite and > 0, alignment, outputs
 * overlapping nothing, workspace size).  Makes no HIP call and dereferences
 * nothing.  sattn_bwd_query and sattn_bwd_key apply the parts that concern
 * their own arguments.
 */
int sattn_bwd_check(const void* Q, const void* K, const void* Vt, const void* O, const void* dO,
                    const float* L, const float* dQ, const float* dK, const float* dVt,
                    const float* D, const void* workspace, unsigned long long workspace_bytes,
                    float c, float s, int T, int Hq, int Hkv);

/* sattn_bwd_query_check, sattn_bwd_key_check: the validation that
 * sattn_bwd_query and sattn_bwd_key apply to their own arguments (the parts
 * of sattn_bwd_check that concern them).  No HIP call, no dereference. */
int sattn_bwd_query_check(const void* Q, const void* K, const void* Vt, const void* O,
                          const void* dO, const float* L, const float* dQ, const float* D,
                          float c, float s, int T, int Hq, int Hkv);
int sattn_bwd_key_check(const void* Q, const void* K, const void* Vt, const void* dO,
                        const float* L, const float* D, const float* dK, const float* dVt,
                        const void* workspace, unsigned long long workspace_bytes, float c,
                        float s, int T, int Hq, int Hkv);

/*
 * sattn_mat_fwd: the materialised causal attention, the baseline the
 * streaming forward avoids (the pages' materialised path: the Graph page's
 * scores plane cgScores, 4*H*T^2 bytes, and its binary16 variant; the causal
 * softmax device image; probabilities rounded to binary16 before their
 * product with V).  Three launches on `stream`:
 *   S[h][i][j] = c (q_i . k_j)                  binary32, base-2 units
 *   L[h][i]    = log2 sum_{j<=i} 2^S[h][i][j]   binary32
 *   P[h][i][j] = 2^(S[h][i][j] - L[h][i])       rounded to binary16
 *   O[i][h*64+d] = sum_{j<=i} P[h][i][j] V_j[d] binary32 sums, binary16 result
 * for keys j <= i.
 *   Q, K, Vt, O, L  as for sattn_fwd (O and L: every element written)
 *   S   device, binary32 [Hq][T][T]: elements with j <= i are written, the
 *       others are neither written nor used
 *   P   device, binary16 [Hq][T][T]: likewise
 * S and P are caller-owned planes (16-byte aligned) that may not overlap
 * anything else; Hq * T * T * 4 must not exceed 2^40.  Validation as
 * sattn_fwd plus those planes; asynchronous like sattn_fwd.
 */
int sattn_mat_fwd(const void* Q, const void* K, const void* Vt, void* O, float* L, float* S,
                  void* P, float c, int T, int Hq, int Hkv, void* stream);

/* sattn_mat_fwd_check: the validation of sattn_mat_fwd alone (no HIP call). */
int sattn_mat_fwd_check(const void* Q, const void* K, const void* Vt, const void* O,
                        const float* L, const float* S, const void* P, float c, int T, int Hq,
                        int Hkv);

/*
 * The three launches of sattn_mat_fwd, one at a time (enqueue them in this
 * order on one stream): sattn_mat_scores writes S; sattn_mat_softmax reads S
 * and writes P and L; sattn_mat_pv reads P and V^T and writes O.  Arguments
 * and layouts as for sattn_mat_fwd; each validates its own (the *_check
 * functions, no HIP call) before enqueueing anything.
 */
int sattn_mat_scores(const void* Q, const void* K, float* S, float c, int T, int Hq, int Hkv,
                     void* stream);
int sattn_mat_softmax(const float* S, void* P, float* L, int T, int Hq, void* stream);
int sattn_mat_pv(const void* P, const void* Vt, void* O, int T, int Hq, int Hkv, void* stream);
int sattn_mat_scores_check(const void* Q, const void* K, const float* S, float c, int T, int Hq,
                           int Hkv);
int sattn_mat_softmax_check(const float* S, const void* P, const float* L, int T, int Hq);
int sattn_mat_pv_check(const void* P, const void* Vt, const void* O, int T, int Hq, int Hkv);

/* sattn_status_string: a static, NUL-terminated description of a status code
 * (an unknown code gives "unknown sattn status").  Never NULL. */
const char* sattn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SATTN_H */
