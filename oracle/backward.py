"""Float64 CPU oracle for the backward of causal streaming attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes (StreamingAttentionSM86 page, the comment that opens the
backward pass, and the comments of its query and key launches): with the
forward's base-2 log-sum-exp L and output O given as inputs, and the output
gradient dO,

    P_ij  = 2^(c (q_i . k_j) - L_i)        for keys j <= i, else 0
    dP_ij = dO_i . v_j
    D_i   = sum_d dO_id O_id                (the row term, from the given O)
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = s sum_j dS_ij k_j
    dK_j  = s sum_i dS_ij q_i               (summed over the query heads of
    dV_j  =   sum_i P_ij dO_i                the K/V head's group)

with c the base-2 and s the natural score scale (the query launch's last two
parameters).  When O and L are the exact forward results and c = s log2(e),
dQ, dK and dV are the exact gradients of sum(dO * O) with respect to Q, K and
V.  The oracle is this definition in float64: P is recomputed from the given
L (not renormalised), D uses the given O, and neither the binary16 rounding of
P and dS nor any tiling is modelled.  Query blocks below only bound memory.

Layouts follow the forward: Q [Hq][T][64], K [Hkv][T][64], V^T [Hkv][64][T],
O and dO token-major [T][Hq*64], L and D [Hq][T].  dK is [Hkv][T][64]; the V
gradient is returned transposed like V^T, [Hkv][64][T].  Query head h belongs
to K/V head h // G with G = Hq / Hkv.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 64


def _check(Q, K, Vt, O, dO, L):
    Q, K, Vt = np.asarray(Q), np.asarray(K), np.asarray(Vt)
    O, dO, L = np.asarray(O), np.asarray(dO), np.asarray(L)
    if Q.ndim != 3 or K.ndim != 3 or Vt.ndim != 3:
        raise ValueError("Q, K: [head][T][64]; Vt: [head][64][T]")
    Hq, T, D = Q.shape
    Hkv = K.shape[0]
    if D != HEAD_DIM or K.shape != (Hkv, T, D) or Vt.shape != (Hkv, D, T):
        raise ValueError(f"shape mismatch Q{Q.shape} K{K.shape} Vt{Vt.shape}")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    if O.shape != (T, Hq * D) or dO.shape != (T, Hq * D) or L.shape != (Hq, T):
        raise ValueError(f"shape mismatch O{O.shape} dO{dO.shape} L{L.shape}")
    return Q, K, Vt, O, dO, L, Hq, Hkv, T


def row_terms_ref(O, dO, Hq: int):
    """D [Hq][T] in float64: D[h][i] = sum_d dO[i][h*64+d] * O[i][h*64+d]."""
    O = np.asarray(O, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    T = O.shape[0]
    return (O * dO).reshape(T, Hq, HEAD_DIM).sum(axis=2).T.copy()


def _head(h, Q, K, Vt, O, dO, L, Hq, Hkv):
    """float64 operands of query head h: q, k, v ([T][64] each), do, o, l."""
    kv = h // (Hq // Hkv)
    cols = slice(h * HEAD_DIM, (h + 1) * HEAD_DIM)
    return (kv, Q[h].astype(np.float64), K[kv].astype(np.float64),
            Vt[kv].astype(np.float64).T, dO[:, cols].astype(np.float64),
            O[:, cols].astype(np.float64), L[h].astype(np.float64))


def _tile(q, k, v, do, Dh, l, c, i0, i1):
    """P and dS of query rows i0..i1-1 against keys 0..i1-1 (masked keys 0)."""
    t = (q[i0:i1] @ k[:i1].T) * c
    rows = np.arange(i0, i1)[:, None]
    cols = np.arange(i1)[None, :]
    t[cols > rows] = -np.inf                     # key j visible to query i iff j <= i
    P = np.exp2(t - l[i0:i1, None])
    dP = do[i0:i1] @ v[:i1].T
    dS = P * (dP - Dh[i0:i1, None])
    return P, dS


def attention_backward_ref(Q, K, Vt, O, dO, L, c, s, *, block: int = 256):
    """The backward in float64.

    Returns ``(dQ, dK, dVt, D)``: dQ ``[Hq][T][64]``, dK ``[Hkv][T][64]``,
    dVt ``[Hkv][64][T]`` (the V gradient, transposed like V^T) and the row
    term D ``[Hq][T]``.
    """
    Q, K, Vt, O, dO, L, Hq, Hkv, T = _check(Q, K, Vt, O, dO, L)
    c, s = float(c), float(s)
    D = row_terms_ref(O, dO, Hq)
    dQ = np.zeros((Hq, T, HEAD_DIM))
    dK = np.zeros((Hkv, T, HEAD_DIM))
    dV = np.zeros((Hkv, T, HEAD_DIM))
    for h in range(Hq):
        kv, q, k, v, do, _, l = _head(h, Q, K, Vt, O, dO, L, Hq, Hkv)
        for i0 in range(0, T, block):
            i1 = min(T, i0 + block)
            P, dS = _tile(q, k, v, do, D[h], l, c, i0, i1)
            dQ[h, i0:i1] = s * (dS @ k[:i1])
            dK[kv, :i1] += s * (dS.T @ q[i0:i1])
            dV[kv, :i1] += P.T @ do[i0:i1]
    return dQ, dK, np.ascontiguousarray(dV.transpose(0, 2, 1)), D


def backward_query_rows_ref(Q, K, Vt, O, dO, L, c, s, h: int, rows):
    """dQ and D of selected query rows of head h, with their P and dS rows.

    Returns a dict: ``dQ`` [n][64], ``D`` [n], ``P`` and ``dS`` [n][T]
    (zero for keys after the row).  Used at sizes where the full oracle would
    take too long, and to derive error bounds from the exact intermediates.
    """
    Q, K, Vt, O, dO, L, Hq, Hkv, T = _check(Q, K, Vt, O, dO, L)
    c, s = float(c), float(s)
    _, q, k, v, do, o, l = _head(h, Q, K, Vt, O, dO, L, Hq, Hkv)
    rows = list(rows)
    out = {"dQ": np.empty((len(rows), HEAD_DIM)), "D": np.empty(len(rows)),
           "P": np.zeros((len(rows), T)), "dS": np.zeros((len(rows), T))}
    for n, i in enumerate(rows):
        Di = float(do[i] @ o[i])
        t = (k[:i + 1] @ q[i]) * c
        P = np.exp2(t - l[i])
        dS = P * (v[:i + 1] @ do[i] - Di)
        out["dQ"][n] = s * (dS @ k[:i + 1])
        out["D"][n] = Di
        out["P"][n, :i + 1] = P
        out["dS"][n, :i + 1] = dS
    return out


def backward_key_rows_ref(Q, K, Vt, O, dO, L, c, s, kv: int, keys):
    """dK and dV rows of selected keys of K/V head kv, with their P and dS
    columns for every query head of the group.

    Returns a dict: ``dK`` and ``dV`` [n][64], ``P`` and ``dS`` [G][T][n]
    (zero for queries before the key).
    """
    Q, K, Vt, O, dO, L, Hq, Hkv, T = _check(Q, K, Vt, O, dO, L)
    c, s = float(c), float(s)
    G = Hq // Hkv
    keys = list(keys)
    out = {"dK": np.zeros((len(keys), HEAD_DIM)), "dV": np.zeros((len(keys), HEAD_DIM)),
           "P": np.zeros((G, T, len(keys))), "dS": np.zeros((G, T, len(keys)))}
    for z in range(G):
        h = kv * G + z
        _, q, k, v, do, o, l = _head(h, Q, K, Vt, O, dO, L, Hq, Hkv)
        Dh = (do * o).sum(axis=1)                 # the row terms of head h
        for n, j in enumerate(keys):
            t = (q[j:] @ k[j]) * c                # queries i >= j see key j
            P = np.exp2(t - l[j:])
            dS = P * (do[j:] @ v[j] - Dh[j:])
            out["dK"][n] += s * (dS @ q[j:])
            out["dV"][n] += P @ do[j:]
            out["P"][z, j:, n] = P
            out["dS"][z, j:, n] = dS
    return out
