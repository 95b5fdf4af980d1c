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
