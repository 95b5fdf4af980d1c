"""Parity on a fixed list of seeded random shapes: sequence lengths from 1 to
6000 (ragged tails of every size), one to 32 K/V heads, groups of 1, 2,
3, 4, 5 or 8 query heads, and the value distributions of the synthetic
workloads.  Each shape runs through both
entries (V^T and V as rows) on whichever kernel its grid selects; the two must
agree bit for bit, and the result must match the float64 oracle (in full where
that takes seconds, on sampled rows of every head otherwise).
"""
import numpy as np
import pytest

from causal_attention_forward_amd.inputs import make_inputs
from oracle import attention_ref, attention_rows_ref
from parity_util import TOL_L, TOL_O, assert_close, note, sample_rows

pytestmark = pytest.mark.gpu


def random_shapes(seed=2024):
    """Ten short shapes (T drawn log-uniformly in [1, 600]: the split-key
    kernel) and ten long, many-headed ones (T uniform in [2000, 6000]: mostly
    the eight-wave kernel)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(20):
        kw = {"qk_std": float(rng.choice([0.5, 1.0, 1.5])),
              "peaked_fraction": float(rng.choice([0.0, 0.01]))}
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        if i < 10:
            T = max(1, int(np.exp(rng.uniform(0.0, np.log(600.0)))))
            Hkv = int(rng.choice([1, 2, 4, 8]))
        else:
            T = int(rng.integers(2000, 6001))
            Hkv = int(rng.choice([8, 16, 32]))
        out.append((T, Hkv * G, Hkv, 300 + i, kw))
    return out


SHAPES = random_shapes()


@pytest.mark.parametrize("T,Hq,Hkv,seed,kw", SHAPES,
                         ids=[f"T{t}_Hq{q}_Hkv{k}" for t, q, k, _, _ in SHAPES])
def test_random_shape(sattn, dev, T, Hq, Hkv, seed, kw):
    import torch
    note(f"random shape T={T} Hq={Hq} Hkv={Hkv} {kw}")
    x = make_inputs(T, Hq, Hkv, seed=seed, **kw)
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    v = torch.from_numpy(np.ascontiguousarray(x.Vt.transpose(0, 2, 1))).to(dev)
    O, L = sattn.fwd(q, k, vt, x.c)
    O2, L2 = sattn.fwd_vrows(q, k, v, x.c)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(L, L2), "V^T and V-rows entries differ"
    Og, Lg = O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64)
    if T * Hq <= 1000 * 16:
        Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
        assert_close(Og, Lg, Or, Lr, f"T={T} Hq={Hq} Hkv={Hkv}")
        return
    rng = np.random.default_rng(seed)
    for h in range(Hq):
        rows = sample_rows(T, rng, extra=4)
        Or, Lr = attention_rows_ref(x.Q, x.K, x.Vt, x.c, h, rows)
        eo = np.abs(Og[rows, h * 64:(h + 1) * 64] - Or).max()
        el = np.abs(Lg[h, rows] - Lr).max()
        assert eo <= TOL_O and el <= TOL_L, f"head {h}: max|dO|={eo} max|dL|={el}"
