"""Float64 CPU oracle for the causal streaming-attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes (StreamingAttentionSM86 page, header comment of the forward
realization): for every query head h and query row i, the causal softmax of
the base-2 scores t_ij = c * (q_i . k_j) over keys j <= i (the diagonal is
kept, per the page's diagonal-tile mask comment), applied to V, and the base-2
log-sum-exp of the same scores.  The streaming method folds a running maximum,
sum and weighted sum tile by tile; that fold is an exact rewrite of this
materialised definition (the page's merge rule for normalised weighted sums),
so the oracle is the definition itself, in float64, with no tiling of the
softmax and no modelling of the binary16 rounding of P or of the hardware
exp2.  Query blocks below only bound memory: each row's softmax is taken over
its whole key range at once.

Head map: query head h reads K/V head h // G with G = Hq / Hkv (the page
numbers the query heads kvHead * groups + z).  Output O is token-major
``[T][Hq*64]`` (heads merged) and L is ``[Hq][T]``.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 64


def _check(Q, K, Vt):
    Q = np.asarray(Q)
    K = np.asarray(K)
    Vt = np.asarray(Vt)
    if Q.ndim != 3 or K.ndim != 3 or Vt.ndim != 3:
        raise ValueError("Q, K: [head][T][64]; Vt: [head][64][T]")
    Hq, T, D = Q.shape
    Hkv = K.shape[0]
    if D != HEAD_DIM or K.shape != (Hkv, T, D) or Vt.shape != (Hkv, D, T):
        raise ValueError(f"shape mismatch Q{Q.shape} K{K.shape} Vt{Vt.shape}")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return Q, K, Vt, Hq, Hkv, T


def attention_ref(Q, K, Vt, c, *, heads=None, block: int = 256):
    """Materialised causal attention in float64.

    Returns ``(O, L)``: O float64 ``[T][Hq*64]`` (token-major, heads merged),
    L float64 ``[Hq][T]`` (base-2 log-sum-exp of t_ij over j <= i).  Heads not
    listed in ``heads`` are left as NaN.
    """
    Q, K, Vt, Hq, Hkv, T = _check(Q, K, Vt)
    G = Hq // Hkv
    c = float(c)
    O = np.full((T, Hq * HEAD_DIM), np.nan)
    L = np.full((Hq, T), np.nan)
    for h in (range(Hq) if heads is None else heads):
        kv = h // G
        q = Q[h].astype(np.float64)
        k = K[kv].astype(np.float64)
        v = Vt[kv].astype(np.float64).T          # V[j][d] = Vt[kv][d][j]
        for i0 in range(0, T, block):
            i1 = min(T, i0 + block)
            t = (q[i0:i1] @ k[:i1].T) * c        # base-2 scores of keys 0..i1-1
            rows = np.arange(i0, i1)[:, None]
            cols = np.arange(i1)[None, :]
            t[cols > rows] = -np.inf             # key j visible to query i iff j <= i
            M = t.max(axis=1, keepdims=True)
            w = np.exp2(t - M)
            Z = w.sum(axis=1, keepdims=True)
            O[i0:i1, h * HEAD_DIM:(h + 1) * HEAD_DIM] = (w @ v[:i1]) / Z
            L[h, i0:i1] = (M + np.log2(Z))[:, 0]
    return O, L


def attention_rows_ref(Q, K, Vt, c, h: int, rows, *, key_chunk: int | None = None):
    """The same definition for selected rows of one query head.

    Returns ``(O_rows, L_rows)``: float64 ``[len(rows)][64]`` and
    ``[len(rows)]``; used to check sampled outputs at sizes where the full
    oracle would take too long.  With ``key_chunk``, the float64 copies of K
    and V are made ``key_chunk`` keys at a time (the scores of every key are
    still formed before the row's maximum and sum are taken), so rows with
    millions of visible keys fit in memory; the arithmetic is unchanged.
    """
    Q, K, Vt, Hq, Hkv, T = _check(Q, K, Vt)
    kv = h // (Hq // Hkv)
    c = float(c)
    rows = list(rows)
    O = np.empty((len(rows), HEAD_DIM))
    L = np.empty(len(rows))
    if key_chunk is None:
        for n, i in enumerate(rows):
            q = Q[h, i].astype(np.float64)
            t = (K[kv, :i + 1].astype(np.float64) @ q) * c
            M = t.max()
            w = np.exp2(t - M)
            Z = w.sum()
            O[n] = (Vt[kv, :, :i + 1].astype(np.float64) @ w) / Z
            L[n] = M + np.log2(Z)
        return O, L
    if len(rows) == 0:
        return O, L
    n_keys = max(rows) + 1
    q = Q[h, rows].astype(np.float64)                       # [R][64]
    t = np.empty((len(rows), n_keys))
    for a in range(0, n_keys, key_chunk):
        b = min(n_keys, a + key_chunk)
        t[:, a:b] = (q @ K[kv, a:b].astype(np.float64).T) * c
    t[np.arange(n_keys)[None, :] > np.asarray(rows)[:, None]] = -np.inf   # keys j <= i only
    M = t.max(axis=1, keepdims=True)
    w = np.exp2(t - M)
    del t
    Z = w.sum(axis=1)
    acc = np.zeros((len(rows), HEAD_DIM))
    for a in range(0, n_keys, key_chunk):
        b = min(n_keys, a + key_chunk)
        acc += w[:, a:b] @ Vt[kv, :, a:b].astype(np.float64).T
    O[:] = acc / Z[:, None]
    L[:] = M[:, 0] + np.log2(Z)
    return O, L


def materialised_rows_ref(Q, K, Vt, c, h: int, rows):
    """The materialised path's intermediate planes for selected rows of head h.

    Returns ``(S_rows, P_rows)``, float64 ``[len(rows)][T]``: the base-2 scores
    S_ij = c (q_i . k_j) and the causal softmax probabilities
    P_ij = 2^(S_ij - M_i) / sum_j' 2^(S_ij' - M_i) for keys j <= i (M_i the row
    maximum); entries with j > i are -inf and 0.  O = P V and L = M + log2 of
    that sum are ``attention_ref``'s results for the same rows.
    """
    Q, K, Vt, Hq, Hkv, T = _check(Q, K, Vt)
    kv = h // (Hq // Hkv)
    c = float(c)
    rows = list(rows)
    S = np.full((len(rows), T), -np.inf)
    P = np.zeros((len(rows), T))
    k = K[kv].astype(np.float64)
    for n, i in enumerate(rows):
        t = (k[:i + 1] @ Q[h, i].astype(np.float64)) * c
        w = np.exp2(t - t.max())
        S[n, :i + 1] = t
        P[n, :i + 1] = w / w.sum()
    return S, P
