"""The backward's error bounds (bwd_util) on the CPU: a NumPy model of the HIP
path's rounding (binary32 products and sums, P and dS rounded to binary16 as
product operands) stays inside them, and a planted indexing mistake in that
model does not.  This checks the tolerance itself, not the HIP code."""
import numpy as np

from bwd_util import Case, key_rows_expected, query_rows_expected

f32, f16 = np.float32, np.float16


def model(case, shift=0):
    """dQ, dK, dV (V gradient untransposed) and D with the HIP path's rounding;
    ``shift`` moves the causal mask (a planted mistake when nonzero)."""
    x = case.x
    T, Hq, Hkv, G = case.T, case.Hq, case.Hkv, case.G
    c, s = f32(case.c), f32(case.s)
    dQ = np.zeros((Hq, T, 64), f32)
    dK = np.zeros((Hkv, T, 64), f32)
    dV = np.zeros((Hkv, T, 64), f32)
    D = np.zeros((Hq, T), f32)
    mask = np.arange(T)[None, :] > np.arange(T)[:, None] + shift
    for h in range(Hq):
        kv = h // G
        q = x.Q[h].astype(f32)
        k = x.K[kv].astype(f32)
        v = x.Vt[kv].astype(f32).T
        do = case.dO[:, h * 64:(h + 1) * 64].astype(f32)
        o = case.O[:, h * 64:(h + 1) * 64].astype(f32)
        D[h] = (do * o).sum(axis=1, dtype=f32)
        S = (q @ k.T).astype(f32)
        S[mask] = -np.inf
        P = np.exp2(S * c - case.L[h][:, None]).astype(f32)
        dS = (P * ((do @ v.T).astype(f32) - D[h][:, None])).astype(f32)
        P16, dS16 = P.astype(f16).astype(f32), dS.astype(f16).astype(f32)
        dQ[h] = s * (dS16 @ k)
        dK[kv] += s * (dS16.T @ q)
        dV[kv] += P16.T @ do
    return dQ, dK, dV, D


def worst_ratio(case, got):
    dQ, dK, dV, D = got
    rows = list(range(case.T))
    r = 0.0
    for h in range(case.Hq):
        want, tol, Dw, Dtol = query_rows_expected(case, h, rows)
        r = max(r, float((np.abs(dQ[h] - want) / tol).max()), float((np.abs(D[h] - Dw) / Dtol).max()))
    for kv in range(case.Hkv):
        wk, tk, wv, tv = key_rows_expected(case, kv, rows)
        r = max(r, float((np.abs(dK[kv] - wk) / tk).max()), float((np.abs(dV[kv] - wv) / tv).max()))
    return r


def test_rounding_model_within_bounds():
    for args in ((200, 4, 2, 61), (150, 2, 1, 62)):
        case = Case(*args, qk_std=1.5)
        with np.errstate(invalid="ignore"):
            ratio = worst_ratio(case, model(case))
        assert ratio <= 1.0, ratio   # few-term rows reach about 2/3 (one rounding)


def test_planted_mask_error_exceeds_bounds():
    case = Case(200, 4, 2, 63)
    with np.errstate(invalid="ignore"):
        assert worst_ratio(case, model(case, shift=1)) > 10.0
        assert worst_ratio(case, model(case, shift=-1)) > 10.0
