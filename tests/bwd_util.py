"""Shared pieces of the backward parity tests: seeded inputs, running the HIP
backward through the binding, and element-wise error bounds derived from the
arithmetic of the HIP path.

Inputs (the recipe of the design notes): Q, K, V^T from the forward's seeded
generator, dO from ``make_output_gradient`` (token-major, binary16), and the
forward's O and L from the float64 oracle, rounded to binary16 and binary32
(never from the HIP path); c is the binary32 base-2 scale and s = 1/8 the
natural one.  Both sides consume exactly these arrays.

Bounds.  The HIP path differs from the float64 definition by
  * binary16 rounding of the product operands dS (for dQ and dK) and P (for
    dV): relative 2^-11, or absolute 2^-25 in the subnormal range;
  * binary32 error in dP and D before dS = P (dP - D) is formed: at most
    2^-20 (sum_d |dO_d V_d| + sum_d |dO_d O_d|) per element, times P;
  * binary32 error of P itself (the score sum and the hardware exp2): well
    under 2^-19 relative, covered by taking 1.5 x 2^-11 for the rounding;
  * binary32 accumulation: (n/16 + 32 + G) 2^-24 of the sum of |terms| for an
    n-term sum on the matrix cores followed by the G-plane group sum.
For an output y = sum_j a_j x_j with operand errors e_j the bound is
sum_j (e_j + gamma |a_j|) |x_j|, evaluated in float64 from the oracle's exact
P and dS.  D is a 64-term binary32 sum of exact products: 64 2^-24 of
sum_d |dO_d O_d|.
"""
import math

import numpy as np

from causal_attention_forward_amd.inputs import SCALE_C, make_inputs, make_output_gradient
from oracle import attention_ref, backward_key_rows_ref, backward_query_rows_ref

S_NAT = 0.125
U16 = 2.0 ** -11
SUB16 = 2.0 ** -25
DP_REL = 2.0 ** -20


class Case:
    """One seeded backward input set (numpy, float16 / float32)."""

    def __init__(self, T, Hq, Hkv, seed, **kw):
        self.x = make_inputs(T, Hq, Hkv, seed, **kw)
        self.dO = make_output_gradient(T, Hq, seed)
        O, L = attention_ref(self.x.Q, self.x.K, self.x.Vt, self.x.c)
        self.O = O.astype(np.float16)
        self.L = L.astype(np.float32)
        self.c = float(SCALE_C)
        self.s = S_NAT
        self.T, self.Hq, self.Hkv = T, Hq, Hkv
        self.G = Hq // Hkv

    def args(self):
        return (self.x.Q, self.x.K, self.x.Vt, self.O, self.dO, self.L, self.c, self.s)


def run_bwd(sattn, dev, case):
    """(dQ, dK, dVt, D) from the HIP path as float64 numpy arrays."""
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    x = case.x
    dQ, dK, dVt, D = sattn.bwd(t(x.Q), t(x.K), t(x.Vt), t(case.O), t(case.dO), t(case.L),
                               case.c, case.s)
    torch.cuda.synchronize()
    return tuple(a.cpu().numpy().astype(np.float64) for a in (dQ, dK, dVt, D))


def _gamma(n, G):
    return (n / 16.0 + 32.0 + G) * 2.0 ** -24


def query_rows_expected(case, h, rows):
    """Oracle dQ and D rows of head h with their bounds."""
    x = case.x
    r = backward_query_rows_ref(*case.args(), h, rows)
    kv = h // case.G
    K = np.abs(x.K[kv].astype(np.float64))
    V = np.abs(x.Vt[kv].astype(np.float64).T)
    cols = slice(h * 64, (h + 1) * 64)
    dO = np.abs(case.dO[rows, cols].astype(np.float64))
    O = np.abs(case.O[rows, cols].astype(np.float64))
    P, dS = r["P"], r["dS"]
    seen = (np.arange(case.T)[None, :] <= np.asarray(rows)[:, None]).astype(np.float64)
    B = (dO * O).sum(axis=1) + np.abs(r["D"])
    E = (1.5 * U16 + _gamma(case.T, 1)) * np.abs(dS) + DP_REL * P * (dO @ V.T + B[:, None]) \
        + SUB16 * seen
    tol_dQ = case.s * (E @ K) + 1e-7
    tol_D = 64 * 2.0 ** -24 * (dO * O).sum(axis=1) + 1e-7
    return r["dQ"], tol_dQ, r["D"], tol_D


def key_rows_expected(case, kv, keys):
    """Oracle dK and dV rows of K/V head kv with their bounds."""
    x = case.x
    r = backward_key_rows_ref(*case.args(), kv, keys)
    G, T = case.G, case.T
    Vk = np.abs(x.Vt[kv][:, keys].astype(np.float64).T)          # [n][64]
    g = _gamma(T, G)
    tol_dK = np.zeros((len(keys), 64))
    tol_dV = np.zeros((len(keys), 64))
    seen = (np.arange(T)[:, None] >= np.asarray(keys)[None, :]).astype(np.float64)   # [T][n]
    for z in range(G):
        h = kv * G + z
        cols = slice(h * 64, (h + 1) * 64)
        Qa = np.abs(x.Q[h].astype(np.float64))
        dO = np.abs(case.dO[:, cols].astype(np.float64))
        O = np.abs(case.O[:, cols].astype(np.float64))
        P, dS = r["P"][z], r["dS"][z]                                # [T][n]
        D = (case.dO[:, cols].astype(np.float64) * case.O[:, cols].astype(np.float64)).sum(axis=1)
        B = (dO * O).sum(axis=1) + np.abs(D)
        E = (1.5 * U16 + g) * np.abs(dS) + DP_REL * P * (dO @ Vk.T + B[:, None]) + SUB16 * seen
        tol_dK += case.s * (E.T @ Qa)
        tol_dV += ((1.5 * U16 + g) * P + SUB16 * seen).T @ dO
    return r["dK"], tol_dK + 1e-7, r["dV"], tol_dV + 1e-7


def check_within(got, want, tol, what, note):
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - want)
    ratio = float((err / tol).max())
    note(f"  {what}: max|err|={float(err.max()):.3e} max err/bound={ratio:.3f}")
    assert ratio <= 1.0, f"{what}: error {float(err.max())} exceeds its bound (ratio {ratio})"


def natural_scale_ok():
    """c and s describe the same scale to binary32 accuracy."""
    return abs(float(SCALE_C) * math.log(2.0) - S_NAT) < 1e-8
