"""The largest admitted problem: Hq * 64 * T * 4 <= 2^32 - 1 (the admission
rule), here T = 131071 (ragged: not a multiple of 64) with Hq = 128, Hkv = 8,
just under the bound (2^32 - 2^15).  The whole-tensor sizes reach their
largest values: O and the forward's Q planes hold 2^31 - 2^14 bytes, the
backward's binary32 dQ 2^32 - 2^15, so every offset into them past 2^31 is
taken.  (The per-head buffer offsets scale with T alone and peak at Hq = 1
with the largest T; test_parity_main covers that case.)

Inputs: one head of Q, K, V, dO (and O) is drawn at full length from the
seeded generator; the other heads are distinct cyclic shifts of it along the
tokens (head h of Q shifted by 3h + 1, K/V head kv by 5kv + 2 and 11kv + 3,
...), so every head differs (a head mix-up is still caught).  The full-size
arrays are assembled on the device (exact copies, torch.roll) and the heads
the oracle evaluates are rebuilt on the host by the same shifts.

Forward: sampled rows of three heads against the float64 oracle (rows near
the end span 131071 keys).  Backward: the oracle cannot form the exact O and
L at this size, and the backward's definition takes them as given inputs, so
the test supplies seeded synthetic ones: O drawn like V, and L_i = c |q_i|
max_{j<=i} |k_j| + log2(i + 1), an upper bound of the log-sum-exp that keeps
P <= 1.  Both sides consume exactly those arrays; sampled query rows (dQ, D)
and keys (dK, dV) are compared within the derived bounds of bwd_util.
"""
import numpy as np
import pytest

from causal_attention_forward_amd.inputs import make_inputs, make_output_gradient
from oracle import attention_rows_ref
from parity_util import TOL_L, TOL_O, note

pytestmark = pytest.mark.gpu

T, HQ, HKV = 131071, 128, 8


def test_admission_bound_is_reached():
    assert HQ * 64 * T * 4 <= 2 ** 32 - 1 < HQ * 64 * (T + 1) * 4 + 2 ** 15


SHIFT_Q = lambda h: 3 * h + 1      # noqa: E731  token shift of query head h
SHIFT_K = lambda kv: 5 * kv + 2    # noqa: E731
SHIFT_V = lambda kv: 11 * kv + 3   # noqa: E731
SHIFT_DO = lambda h: 7 * h + 1     # noqa: E731
SHIFT_O = lambda h: 13 * h + 5     # noqa: E731


class Big:
    """Full-size device tensors built from a one-head seeded base by cyclic
    token shifts (exact copies), and the same heads rebuilt on the host on
    demand for the oracle."""

    def __init__(self, dev):
        import torch
        base = make_inputs(T, 1, 1, seed=101)
        self.c = base.c
        self.q0, self.k0, self.vt0 = base.Q[0], base.K[0], base.Vt[0]
        self.g0 = make_output_gradient(T, 1, seed=101)
        self.o0 = make_output_gradient(T, 1, seed=102)
        tq, tk, tv = (torch.from_numpy(a).to(dev) for a in (self.q0, self.k0, self.vt0))
        tg, to = (torch.from_numpy(a).to(dev) for a in (self.g0, self.o0))
        self.Q = torch.stack([torch.roll(tq, SHIFT_Q(h), 0) for h in range(HQ)])
        self.K = torch.stack([torch.roll(tk, SHIFT_K(kv), 0) for kv in range(HKV)])
        self.Vt = torch.stack([torch.roll(tv, SHIFT_V(kv), 1) for kv in range(HKV)])
        self.dO = torch.stack([torch.roll(tg, SHIFT_DO(h), 0) for h in range(HQ)], 1).reshape(T, HQ * 64)
        self.O = torch.stack([torch.roll(to, SHIFT_O(h), 0) for h in range(HQ)], 1).reshape(T, HQ * 64)

    # host copies of single heads (the oracle indexes heads, so one-head
    # arrays with the head map of a one-head problem are equivalent)
    def q(self, h):
        return np.roll(self.q0, SHIFT_Q(h), 0)

    def k(self, kv):
        return np.roll(self.k0, SHIFT_K(kv), 0)

    def vt(self, kv):
        return np.roll(self.vt0, SHIFT_V(kv), 1)

    def do(self, h):
        return np.roll(self.g0, SHIFT_DO(h), 0)

    def o(self, h):
        return np.roll(self.o0, SHIFT_O(h), 0)


@pytest.fixture(scope="module")
def big(dev):
    note(f"building inputs T={T} Hq={HQ} Hkv={HKV}")
    x = Big(dev)
    note("inputs ready")
    return x


def test_forward_at_the_size_limit(sattn, dev, big):
    import torch
    x = big
    O, L = sattn.fwd(x.Q, x.K, x.Vt, x.c)
    torch.cuda.synchronize()
    note("forward done")
    rows = [0, 1, 63, 64, 65537, T - 65, T - 2, T - 1]
    for h in (0, 77, HQ - 1):
        kv = h // (HQ // HKV)
        Og = O[rows, h * 64:(h + 1) * 64].cpu().numpy().astype(np.float64)
        Lg = L[h, rows].cpu().numpy().astype(np.float64)
        Or, Lr = attention_rows_ref(x.q(h)[None], x.k(kv)[None], x.vt(kv)[None], x.c, 0, rows)
        eo, el = float(np.abs(Og - Or).max()), float(np.abs(Lg - Lr).max())
        note(f"  head {h}: max|dO|={eo:.3e} max|dL|={el:.3e}")
        assert eo <= TOL_O and el <= TOL_L
    del O, L
    torch.cuda.empty_cache()


def test_backward_at_the_size_limit(sattn, dev, big):
    import torch
    from bwd_util import DP_REL, S_NAT, SUB16, U16, _gamma
    from oracle import backward_key_rows_ref, backward_query_rows_ref
    x = big
    c = float(x.c)
    G = HQ // HKV
    # L_i = c |q_i| max_{j<=i} |k_j| + log2(i+1) >= log2 sum_{j<=i} 2^(c q_i.k_j)
    kn = torch.cummax(x.K.float().norm(dim=2), dim=1).values          # [Hkv][T]
    qn = x.Q.float().norm(dim=2)                                      # [Hq][T]
    pos = torch.log2(torch.arange(1, T + 1, device=dev, dtype=torch.float32))
    L = (c * qn * kn.repeat_interleave(G, 0) * 1.0001 + pos[None, :]).contiguous()
    Lh = L.cpu().numpy()
    note("synthetic L ready")
    dQ, dK, dVt, D = sattn.bwd(x.Q, x.K, x.Vt, x.O, x.dO, L, c, S_NAT)
    torch.cuda.synchronize()
    note("backward done")
    rows = [0, 1, 64, 98303, T - 2, T - 1]
    for h in (0, HQ - 1):
        kv = h // G
        q, k, vt, do, o = x.q(h), x.k(kv), x.vt(kv), x.do(h), x.o(h)
        r = backward_query_rows_ref(q[None], k[None], vt[None], o, do, Lh[h:h + 1], c, S_NAT, 0, rows)
        Ka = np.abs(k.astype(np.float64))
        Va = np.abs(vt.astype(np.float64).T)
        dOa = np.abs(do[rows].astype(np.float64))
        Oa = np.abs(o[rows].astype(np.float64))
        B = (dOa * Oa).sum(axis=1) + np.abs(r["D"])
        seen = (np.arange(T)[None, :] <= np.asarray(rows)[:, None]).astype(np.float64)
        E = (1.5 * U16 + _gamma(T, 1)) * np.abs(r["dS"]) \
            + DP_REL * r["P"] * (dOa @ Va.T + B[:, None]) + SUB16 * seen
        tol = S_NAT * (E @ Ka) + 1e-7
        got = dQ[h, rows].cpu().numpy().astype(np.float64)
        ratio = float((np.abs(got - r["dQ"]) / tol).max())
        note(f"  dQ head {h}: err/bound {ratio:.3f}")
        assert ratio <= 1.0
        Dg = D[h, rows].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(Dg - r["D"]) <= 64 * 2.0 ** -24 * (dOa * Oa).sum(axis=1) + 1e-7)
    keys = [0, T // 2 + 1, T - 1]
    kv = HKV - 1
    heads = range(kv * G, (kv + 1) * G)
    Qg = np.stack([x.q(h) for h in heads])
    dOg = np.concatenate([x.do(h) for h in heads], axis=1)
    Og = np.concatenate([x.o(h) for h in heads], axis=1)
    k, vt = x.k(kv), x.vt(kv)
    r = backward_key_rows_ref(Qg, k[None], vt[None], Og, dOg, Lh[kv * G:(kv + 1) * G], c, S_NAT, 0,
                              keys)
    g = _gamma(T, G)
    Vk = np.abs(vt[:, keys].astype(np.float64).T)
    seen = (np.arange(T)[:, None] >= np.asarray(keys)[None, :]).astype(np.float64)
    tk = np.zeros((len(keys), 64))
    tv = np.zeros((len(keys), 64))
    for z in range(G):
        cols = slice(z * 64, (z + 1) * 64)
        Qa = np.abs(Qg[z].astype(np.float64))
        dOa = np.abs(dOg[:, cols].astype(np.float64))
        Oa = np.abs(Og[:, cols].astype(np.float64))
        Dz = (dOg[:, cols].astype(np.float64) * Og[:, cols].astype(np.float64)).sum(axis=1)
        B = (dOa * Oa).sum(axis=1) + np.abs(Dz)
        P, dS = r["P"][z], r["dS"][z]
        E = (1.5 * U16 + g) * np.abs(dS) + DP_REL * P * (dOa @ Vk.T + B[:, None]) + SUB16 * seen
        tk += S_NAT * (E.T @ Qa)
        tv += ((1.5 * U16 + g) * P + SUB16 * seen).T @ dOa
    gk = dK[kv, keys].cpu().numpy().astype(np.float64)
    gv = dVt[kv][:, keys].cpu().numpy().astype(np.float64).T
    rk = float((np.abs(gk - r["dK"]) / (tk + 1e-7)).max())
    rv = float((np.abs(gv - r["dV"]) / (tv + 1e-7)).max())
    note(f"  dK/dV K/V head {kv}: err/bound {rk:.3f} / {rv:.3f}")
    assert rk <= 1.0 and rv <= 1.0
