"""The largest admitted head count, Hq = 65535 (the admission rule's bound on
query heads), at T = 255 and 250 (the rule's bound on Hq * 64 * T * 4 allows
T <= 256 there).  The eight-wave kernel then runs its largest grids (65535
workgroups), every
per-head offset of Q, O and L is taken up to about 2^31 bytes, and the GQA
extremes are both covered: one K/V head per query head, and all 65535 query
heads on one K/V head (a group of 65535, odd, so one head per workgroup slot
group); T = 250 has a group of 13107 over five K/V heads and a ragged last
tile.

Inputs: one head of Q, K and V^T is drawn from the seeded generator; every
other head is a distinct cyclic shift of it along the tokens (query head h by
3h + 1, K/V head kv by 5kv + 2 and 11kv + 3, modulo T), assembled on the
device by one gather; the heads the oracle evaluates are rebuilt on the host
by the same shifts.  Outputs: finite everywhere, and whole rows of sampled
heads (first, last and two inside) against the float64 oracle; the V-rows
entry bit-identical to the V^T entry on the same values.
"""
import numpy as np
import pytest

from causal_attention_forward_amd.inputs import make_inputs
from oracle import attention_ref
from parity_util import TOL_L, TOL_O, note

HQ = 65535


def test_shapes_are_at_the_head_bound():
    # Hq <= 65535 is its own bound; with it, T <= 256 keeps Hq * 64 * T * 4
    # within 32 bits
    for T in (255, 250, 256):
        assert HQ * 64 * T * 4 <= 2 ** 32 - 1
    assert HQ * 64 * 257 * 4 > 2 ** 32 - 1


def shift_q(h, T):
    return (3 * h + 1) % T


def shift_k(kv, T):
    return (5 * kv + 2) % T


def shift_v(kv, T):
    return (11 * kv + 3) % T


@pytest.mark.gpu
@pytest.mark.parametrize("T,Hkv", [(255, HQ), (255, 1), (250, 5)])
def test_max_heads(sattn, dev, T, Hkv):
    import torch
    note(f"max heads: T={T} Hq={HQ} Hkv={Hkv}")
    base = make_inputs(T, 1, 1, seed=131)
    q0, k0, vt0 = base.Q[0], base.K[0], base.Vt[0]
    t = torch.arange(T, device=dev)

    def rolled(x0, shifts, axis):
        # head i = np.roll(x0, shifts[i], axis): element t comes from (t - shift) mod T
        idx = (t[None, :] - shifts[:, None]) % T
        xd = torch.from_numpy(x0).to(dev)
        return xd[idx] if axis == 0 else xd[:, idx].permute(1, 0, 2).contiguous()

    hs = torch.arange(HQ, device=dev)
    kvs = torch.arange(Hkv, device=dev)
    Q = rolled(q0, (3 * hs + 1) % T, 0)
    K = rolled(k0, (5 * kvs + 2) % T, 0)
    Vt = rolled(vt0, (11 * kvs + 3) % T, 1)
    O, L = sattn.fwd(Q, K, Vt, base.c)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(L).all())
    G = HQ // Hkv
    for h in (0, 1, 40000, HQ - 1):
        kv = h // G
        q = np.roll(q0, shift_q(h, T), 0)[None]
        k = np.roll(k0, shift_k(kv, T), 0)[None]
        vt = np.roll(vt0, shift_v(kv, T), 1)[None]
        Or, Lr = attention_ref(q, k, vt, base.c)
        Og = O[:, h * 64:(h + 1) * 64].cpu().numpy().astype(np.float64)
        Lg = L[h].cpu().numpy().astype(np.float64)
        eo, el = float(np.abs(Og - Or).max()), float(np.abs(Lg - Lr[0]).max())
        note(f"  head {h} (K/V head {kv}): max|dO|={eo:.3e} max|dL|={el:.3e}")
        assert eo <= TOL_O and el <= TOL_L
    V = Vt.transpose(1, 2).contiguous()
    del Vt
    O2, L2 = sattn.fwd_vrows(Q, K, V, base.c)
    torch.cuda.synchronize()
    assert torch.equal(O2, O) and torch.equal(L2, L), "V rows differ from the V^T path"
    del Q, K, V, O, L, O2, L2
    torch.cuda.empty_cache()


@pytest.mark.gpu
@pytest.mark.parametrize("Hkv", [HQ, 1])
def test_max_heads_backward(sattn, dev, Hkv):
    """The backward at Hq = 65535, T = 255: the query launch's dQ plane holds
    65535 * 255 * 64 binary32 (just under 2^32 bytes), so its per-head offsets
    pass 2^31; with one K/V head the grouped reduction sums 65535 planes.  The
    backward takes O and L as given, so they are seeded synthetic arrays (O
    drawn like dO, L_i = c |q_i| max_{j<=i} |k_j| + log2(i + 1), which keeps
    P <= 1), the same on both sides.  dQ and D rows of sampled heads within
    the derived bounds; dK and dV rows of sampled K/V heads where the oracle
    can form them (one query head per K/V head), and with one K/V head the
    last key's dK and dV rows, which only the 65535 heads' last queries
    reach, against their float64 sums over the group."""
    import torch
    from bwd_util import DP_REL, S_NAT, SUB16, U16, _gamma
    from causal_attention_forward_amd.inputs import make_output_gradient
    from oracle import backward_key_rows_ref, backward_query_rows_ref
    T = 255
    note(f"max heads backward: T={T} Hq={HQ} Hkv={Hkv}")
    base = make_inputs(T, 1, 1, seed=132)
    q0, k0, vt0 = base.Q[0], base.K[0], base.Vt[0]
    g0 = make_output_gradient(T, 1, seed=132)
    o0 = make_output_gradient(T, 1, seed=133)
    c = float(base.c)
    t = torch.arange(T, device=dev)
    hs = torch.arange(HQ, device=dev)
    kvs = torch.arange(Hkv, device=dev)

    def gather(x0, shifts):
        return torch.from_numpy(x0).to(dev)[(t[None, :] - shifts[:, None]) % T]

    Q = gather(q0, (3 * hs + 1) % T)
    K = gather(k0, (5 * kvs + 2) % T)
    Vt = torch.from_numpy(vt0).to(dev)[:, (t[None, :] - ((11 * kvs + 3) % T)[:, None]) % T]
    Vt = Vt.permute(1, 0, 2).contiguous()
    dO = gather(g0, (7 * hs + 1) % T).permute(1, 0, 2).reshape(T, HQ * 64).contiguous()
    O = gather(o0, (13 * hs + 5) % T).permute(1, 0, 2).reshape(T, HQ * 64).contiguous()
    G = HQ // Hkv
    kn = torch.cummax(K.float().norm(dim=2), dim=1).values
    qn = Q.float().norm(dim=2)
    pos = torch.log2(torch.arange(1, T + 1, device=dev, dtype=torch.float32))
    kv_of = hs // G
    L = (c * qn * kn[kv_of] * 1.0001 + pos[None, :]).contiguous()
    dQ, dK, dVt, D = sattn.bwd(Q, K, Vt, O, dO, L, c, S_NAT)
    torch.cuda.synchronize()
    for a in (dQ, dK, dVt, D):
        assert bool(torch.isfinite(a).all())
    rows = list(range(T))
    for h in (0, 40000, HQ - 1):
        kv = h // G
        q = np.roll(q0, shift_q(h, T), 0)
        k = np.roll(k0, shift_k(kv, T), 0)
        vt = np.roll(vt0, shift_v(kv, T), 1)
        do = np.roll(g0, (7 * h + 1) % T, 0)
        o = np.roll(o0, (13 * h + 5) % T, 0)
        Lh = L[h:h + 1].cpu().numpy()
        r = backward_query_rows_ref(q[None], k[None], vt[None], o, do, Lh, c, S_NAT, 0, rows)
        Ka = np.abs(k.astype(np.float64))
        Va = np.abs(vt.astype(np.float64).T)
        dOa = np.abs(do.astype(np.float64))
        Oa = np.abs(o.astype(np.float64))
        B = (dOa * Oa).sum(axis=1) + np.abs(r["D"])
        seen = (np.arange(T)[None, :] <= np.arange(T)[:, None]).astype(np.float64)
        E = (1.5 * U16 + _gamma(T, 1)) * np.abs(r["dS"]) \
            + DP_REL * r["P"] * (dOa @ Va.T + B[:, None]) + SUB16 * seen
        tol = S_NAT * (E @ Ka) + 1e-7
        got = dQ[h].cpu().numpy().astype(np.float64)
        ratio = float((np.abs(got - r["dQ"]) / tol).max())
        Dg = D[h].cpu().numpy().astype(np.float64)
        dmax = float(np.abs(Dg - r["D"]).max())
        note(f"  dQ head {h}: err/bound {ratio:.3f}; max|dD| {dmax:.2e}")
        assert ratio <= 1.0
        assert np.all(np.abs(Dg - r["D"]) <= 64 * 2.0 ** -24 * (dOa * Oa).sum(axis=1) + 1e-7)
        if G == 1:
            rk = backward_key_rows_ref(q[None], k[None], vt[None], o, do, Lh, c, S_NAT, 0, rows)
            Qa = np.abs(q.astype(np.float64))
            seenk = seen  # [query][key]: the query at or after the key
            Ek = (1.5 * U16 + _gamma(T, 1)) * np.abs(rk["dS"][0]) \
                + DP_REL * rk["P"][0] * (dOa @ Va.T + B[:, None]) + SUB16 * seenk
            tk = S_NAT * (Ek.T @ Qa) + 1e-7
            tv = ((1.5 * U16 + _gamma(T, 1)) * rk["P"][0] + SUB16 * seenk).T @ dOa + 1e-7
            gk = dK[kv].cpu().numpy().astype(np.float64)
            gv = dVt[kv].cpu().numpy().astype(np.float64).T
            ek = float((np.abs(gk - rk["dK"]) / tk).max())
            ev = float((np.abs(gv - rk["dV"]) / tv).max())
            note(f"  dK/dV K/V head {kv}: err/bound {ek:.3f} / {ev:.3f}")
            assert ek <= 1.0 and ev <= 1.0
    if G > 1:
        # the last key is seen by each head's last query only, so its dK and
        # dV rows are plain sums over the group, summed here in float64
        last = T - 1
        hh = np.arange(HQ)
        qs = q0[(last - (3 * hh + 1)) % T].astype(np.float64)            # [Hq][64]
        dos = g0[(last - (7 * hh + 1)) % T].astype(np.float64)
        os_ = o0[(last - (13 * hh + 5)) % T].astype(np.float64)
        kvv = hh // G
        ks = k0[(last - (5 * kvv + 2)) % T].astype(np.float64)
        vs = vt0[:, (last - (11 * kvv + 3)) % T].T.astype(np.float64)
        Ll = L[:, last].cpu().numpy().astype(np.float64)
        P = np.exp2(c * (qs * ks).sum(axis=1) - Ll)
        dP = (dos * vs).sum(axis=1)
        Dr = (dos * os_).sum(axis=1)
        dS = P * (dP - Dr)
        g = _gamma(T, G)
        for kv in range(Hkv):
            sel = kvv == kv
            want_v = (P[sel, None] * dos[sel]).sum(axis=0)
            want_k = S_NAT * (dS[sel, None] * qs[sel]).sum(axis=0)
            B = (np.abs(dos[sel]) * np.abs(os_[sel])).sum(axis=1) + np.abs(Dr[sel])
            Ek = (1.5 * U16 + g) * np.abs(dS[sel]) \
                + DP_REL * P[sel] * ((np.abs(dos[sel]) * np.abs(vs[sel])).sum(axis=1) + B) + SUB16
            tk = S_NAT * (Ek[:, None] * np.abs(qs[sel])).sum(axis=0) + 1e-7
            tv = (((1.5 * U16 + g) * P[sel] + SUB16)[:, None] * np.abs(dos[sel])).sum(axis=0) + 1e-7
            gk = dK[kv, last].cpu().numpy().astype(np.float64)
            gv = dVt[kv, :, last].cpu().numpy().astype(np.float64)
            ek = float((np.abs(gk - want_k) / tk).max())
            ev = float((np.abs(gv - want_v) / tv).max())
            note(f"  dK/dV of the last key, K/V head {kv} (sum of {G} heads): err/bound {ek:.3f} / {ev:.3f}")
            assert ek <= 1.0 and ev <= 1.0
    del Q, K, Vt, dO, O, L, dQ, dK, dVt, D
    torch.cuda.empty_cache()
