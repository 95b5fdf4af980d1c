"""The materialised path (sattn_mat_fwd and its three launches) through the C
ABI against the float64 oracle.

O and L: the forward's tolerances (4e-3, 2e-4).  The planes, per element:
  S: the binary32 sum of 64 exact binary16 products, times c:
     |S - S_ref| <= (64 2^-24 sum_d |q_d k_d| c) + 2^-24 |S_ref|;
  P: binary16 rounding of 2^(S - L) whose exponent is off by at most the S
     error plus the error of L (same order, plus 2^-20 for the sum and log2):
     |P - P_ref| <= P_ref (2^-11 + 2 ln2 (eS_row + 2^-19)) + 2^-25.
Elements above the diagonal are neither written (the planes are filled with a
sentinel first) nor used.
"""
import math

import numpy as np
import pytest

from causal_attention_forward_amd.inputs import make_inputs, make_workload
from oracle import attention_ref, attention_rows_ref, materialised_rows_ref
from parity_util import TOL_L, TOL_O, assert_close, note, sample_rows

pytestmark = pytest.mark.gpu

SENTINEL_F32 = np.float32(-12345.5)
SENTINEL_F16 = np.float16(-777.0)


def run_mat(sattn, dev, x):
    import torch
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    S = torch.full((x.Hq, x.T, x.T), float(SENTINEL_F32), dtype=torch.float32, device=dev)
    P = torch.full((x.Hq, x.T, x.T), float(SENTINEL_F16), dtype=torch.float16, device=dev)
    O, L, S, P = sattn.mat_fwd(q, k, vt, x.c, scores=S, probs=P)
    torch.cuda.synchronize()
    return O, L, S, P


def plane_bounds(x, h, rows, S_ref):
    kv = h // (x.Hq // x.Hkv)
    q = np.abs(x.Q[h, rows].astype(np.float64))
    k = np.abs(x.K[kv].astype(np.float64))
    eS = 64 * 2.0 ** -24 * (q @ k.T) * float(x.c) + 2.0 ** -24 * np.abs(np.where(np.isfinite(S_ref), S_ref, 0))
    return eS


def check_planes(x, S, P, h, rows):
    S_ref, P_ref = materialised_rows_ref(x.Q, x.K, x.Vt, x.c, h, rows)
    Sg = S[h, rows].cpu().numpy().astype(np.float64)
    Pg = P[h, rows].cpu().numpy().astype(np.float64)
    eS = plane_bounds(x, h, rows, S_ref)
    for n, i in enumerate(rows):
        vis = slice(0, i + 1)
        assert np.all(np.abs(Sg[n, vis] - S_ref[n, vis]) <= eS[n, vis]), f"S row {i}"
        tolP = P_ref[n, vis] * (2.0 ** -11 + 2 * math.log(2) * (eS[n, vis].max() + 2.0 ** -19)) \
            + 2.0 ** -25
        assert np.all(np.abs(Pg[n, vis] - P_ref[n, vis]) <= tolP), f"P row {i}"
        assert np.all(Sg[n, i + 1:] == float(SENTINEL_F32)), f"S written above the diagonal, row {i}"
        assert np.all(Pg[n, i + 1:] == float(SENTINEL_F16)), f"P written above the diagonal, row {i}"


# The last two have enough score tiles (at least 16 workgroups per CU) for the
# scores launch's runs of four tiles per workgroup: one aligned, one with
# T % 4 != 0 (element-wise stores) and a ragged last tile.
SHAPES = [(1, 1, 1, {}), (7, 2, 1, {}), (64, 2, 2, {}), (130, 4, 2, {"peaked_fraction": 0.02}),
          (257, 3, 1, {"qk_std": 1.5}), (1000, 16, 4, {"peaked_fraction": 0.01}),
          (1024, 8, 8, {"qk_std": 0.5, "v_std": 0.5}), (1024, 128, 32, {}),
          (999, 112, 8, {"peaked_fraction": 0.01})]


@pytest.mark.parametrize("T,Hq,Hkv,kw", SHAPES, ids=[f"T{t}_Hq{a}_Hkv{b}" for t, a, b, _ in SHAPES])
def test_materialised_full(sattn, dev, T, Hq, Hkv, kw):
    note(f"materialised T={T} Hq={Hq} Hkv={Hkv} {kw}")
    x = make_inputs(T, Hq, Hkv, seed=80 + T % 17, **kw)
    O, L, S, P = run_mat(sattn, dev, x)
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64), Or, Lr,
                 f"T={T}")
    rng = np.random.default_rng(T)
    for h in sorted({0, Hq - 1}):
        check_planes(x, S, P, h, sample_rows(T, rng, extra=6))


def test_materialised_headline_workload_sampled(sattn, dev):
    x = make_workload(3)
    note("materialised T=4096 Hq=32 Hkv=8 (planes 2.1 GB + 1.1 GB), sampled rows")
    O, L, S, P = run_mat(sattn, dev, x)
    Og, Lg = O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(4096)
    for h in (0, 13, 31):
        rows = sample_rows(x.T, rng, extra=6)
        Or, Lr = attention_rows_ref(x.Q, x.K, x.Vt, x.c, h, rows)
        assert np.abs(Og[rows, h * 64:(h + 1) * 64] - Or).max() <= TOL_O
        assert np.abs(Lg[h, rows] - Lr).max() <= TOL_L
        check_planes(x, S, P, h, rows[:12])
    del S, P


def test_three_launches_equal_the_combined_call(sattn, dev):
    import torch
    x = make_inputs(300, 4, 2, seed=90)
    O, L, S, P = run_mat(sattn, dev, x)
    q, k, vt = (torch.from_numpy(a).to(dev) for a in (x.Q, x.K, x.Vt))
    S2 = torch.empty_like(S)
    P2 = torch.zeros_like(P)
    O2 = torch.empty_like(O)
    L2 = torch.empty_like(L)
    st = torch.cuda.current_stream(dev).cuda_stream
    T, Hq, Hkv = x.T, x.Hq, x.Hkv
    assert sattn.sattn_mat_scores(q.data_ptr(), k.data_ptr(), S2.data_ptr(), float(x.c), T, Hq,
                                  Hkv, st) == sattn.SATTN_OK
    assert sattn.sattn_mat_softmax(S2.data_ptr(), P2.data_ptr(), L2.data_ptr(), T, Hq,
                                   st) == sattn.SATTN_OK
    assert sattn.sattn_mat_pv(P2.data_ptr(), vt.data_ptr(), O2.data_ptr(), T, Hq, Hkv,
                              st) == sattn.SATTN_OK
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(L, L2)
    lower = torch.tril(torch.ones(T, T, dtype=torch.bool, device=dev))
    assert torch.equal(S[:, lower], S2[:, lower]) and torch.equal(P[:, lower], P2[:, lower])
