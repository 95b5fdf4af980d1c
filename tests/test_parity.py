"""Parity of the HIP path with the float64 oracle, through the C ABI.

Tolerances (stated for the attention forward): max |O - O_ref| <= 4e-3 and
max |L - L_ref| <= 2e-4 (base-2 units), element by element.  Small and
medium workloads are compared in full; the two largest are compared on
sampled rows of every head (the oracle computes those one by one), plus
properties that hold at any size.
"""
import math

import numpy as np
import pytest

from causal_attention_forward_amd.inputs import WORKLOADS, make_inputs, make_workload
from oracle import attention_ref, attention_rows_ref
from parity_util import TOL_L, TOL_O, assert_close, note, run, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_workload_full(sattn, dev, idx):
    w = WORKLOADS[idx]
    note(f"workload {idx} ({w.name}) full compare")
    x = make_workload(idx)
    O, L = run(sattn, dev, x)
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O, L, Or, Lr, w.name)


@pytest.mark.parametrize("idx", [3, 4])
def test_workload_sampled(sattn, dev, idx):
    w = WORKLOADS[idx]
    note(f"workload {idx} ({w.name}) sampled rows, every head")
    x = make_workload(idx)
    O, L = run(sattn, dev, x)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    # any size: each output is a convex combination of V rows, and L >= the diagonal score
    vmax = np.abs(x.Vt.astype(np.float64)).max(axis=2)          # [Hkv][64]
    G = x.Hq // x.Hkv
    for h in range(x.Hq):
        bound = vmax[h // G] * (1 + 2e-3) + 1e-3
        assert (np.abs(O[:, h * 64:(h + 1) * 64]) <= bound[None, :]).all()
    rng = np.random.default_rng(100 + idx)
    worst_o = worst_l = 0.0
    for h in range(x.Hq):
        rows = sample_rows(x.T, rng)
        Or, Lr = attention_rows_ref(x.Q, x.K, x.Vt, x.c, h, rows)
        worst_o = max(worst_o, float(np.abs(O[rows, h * 64:(h + 1) * 64] - Or).max()))
        worst_l = max(worst_l, float(np.abs(L[h, rows] - Lr).max()))
    note(f"  sampled: max|dO|={worst_o:.3e} max|dL|={worst_l:.3e}")
    assert worst_o <= TOL_O and worst_l <= TOL_L


SHAPES = [(1, 1), (2, 1), (4, 2), (8, 8), (6, 3), (12, 3), (3, 1)]
TS = [1, 2, 3, 7, 8, 9, 31, 33, 63, 64, 65, 96, 127, 128, 129, 200, 255, 257, 1000]


@pytest.mark.parametrize("T", TS)
def test_small_T_sweep(sattn, dev, T):
    note(f"small-T sweep T={T}")
    for j, (hq, hkv) in enumerate(SHAPES):
        x = make_inputs(T, hq, hkv, seed=1000 + 17 * T + j, qk_std=1.25)
        O, L = run(sattn, dev, x)
        Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
        assert_close(O, L, Or, Lr, f"T={T} Hq={hq} Hkv={hkv}")


def test_T1_is_exact(sattn, dev):
    """T=1: P = 2^0 = 1 and l = 1, so O must equal V's first column bit for bit."""
    x = make_inputs(1, 8, 2, seed=5)
    O, L = run(sattn, dev, x)
    for h in range(8):
        assert np.array_equal(O[0, h * 64:(h + 1) * 64], x.Vt[h // 4, :, 0].astype(np.float64))
        t00 = float(x.c) * float(x.Q[h, 0].astype(np.float64) @ x.K[h // 4, 0].astype(np.float64))
        assert abs(L[h, 0] - t00) <= 1e-5 * max(1.0, abs(t00))


@pytest.mark.parametrize("T", [64, 100, 130, 1000])
def test_constant_scores_prefix_mean(sattn, dev, T):
    """Q = 0: O is the prefix mean of V and L = log2(i+1); pins the diagonal
    and the ragged tail on the GPU."""
    x = make_inputs(T, 4, 2, seed=6)
    x.Q[:] = 0
    O, L = run(sattn, dev, x)
    for h in range(4):
        V = x.Vt[h // 2].astype(np.float64).T
        prefix = np.cumsum(V, axis=0) / np.arange(1, T + 1)[:, None]
        assert np.abs(O[:, h * 64:(h + 1) * 64] - prefix).max() <= TOL_O
        assert np.abs(L[h] - np.log2(np.arange(1, T + 1))).max() <= TOL_L


def test_causality_bitwise(sattn, dev):
    """Changing keys and values after row i0 leaves rows 0..i0 bit-identical."""
    x = make_inputs(300, 4, 2, seed=8)
    O1, L1 = run(sattn, dev, x)
    i0 = 150
    rng = np.random.default_rng(3)
    x.K[:, i0 + 1:] = rng.standard_normal(x.K[:, i0 + 1:].shape).astype(np.float16)
    x.Vt[:, :, i0 + 1:] = rng.standard_normal(x.Vt[:, :, i0 + 1:].shape).astype(np.float16)
    O2, L2 = run(sattn, dev, x)
    assert np.array_equal(O1[:i0 + 1], O2[:i0 + 1]) and np.array_equal(L1[:, :i0 + 1], L2[:, :i0 + 1])
    assert not np.array_equal(O1[i0 + 1:], O2[i0 + 1:])


def test_deterministic(sattn, dev):
    x = make_workload(2)
    O1, L1 = run(sattn, dev, x)
    O2, L2 = run(sattn, dev, x)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_guard_bands_untouched(sattn, dev):
    """O and L are written exactly inside their extents: canaries before and
    after both stay intact (ragged T, GQA)."""
    import torch
    T, hq, hkv = 129, 6, 2
    x = make_inputs(T, hq, hkv, seed=9)
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    pad = 4096
    ob = torch.full((pad + T * hq * 64 + pad,), 12345.0, dtype=torch.float16, device=dev)
    lb = torch.full((pad + hq * T + pad,), -777.0, dtype=torch.float32, device=dev)
    O = ob[pad:pad + T * hq * 64].view(T, hq * 64)
    L = lb[pad:pad + hq * T].view(hq, T)
    sattn.fwd(q, k, vt, x.c, out=O, lse=L)
    torch.cuda.synchronize()
    obh = ob.cpu().numpy()
    lbh = lb.cpu().numpy()
    assert (obh[:pad] == np.float16(12345.0)).all() and (obh[-pad:] == np.float16(12345.0)).all()
    assert (lbh[:pad] == -777.0).all() and (lbh[-pad:] == -777.0).all()
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64), Or, Lr,
                 "guarded")


def test_errors_leave_outputs_untouched(sattn, dev):
    import torch
    x = make_inputs(64, 2, 1, seed=10)
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    O = torch.full((64, 128), 3.0, dtype=torch.float16, device=dev)
    L = torch.full((2, 64), 5.0, dtype=torch.float32, device=dev)
    for c in (0.0, -1.0, math.nan, math.inf):
        with pytest.raises(sattn.SattnError):
            sattn.fwd(q, k, vt, c, out=O, lse=L)
    # misaligned Q: same bytes shifted by one element
    qb = torch.zeros(q.numel() + 8, dtype=torch.float16, device=dev)
    st = sattn.sattn_fwd(qb.data_ptr() + 2, k.data_ptr(), vt.data_ptr(), O.data_ptr(), L.data_ptr(),
                         float(x.c), 64, 2, 1, None)
    assert st == sattn.SATTN_ERR_ALIGN
    torch.cuda.synchronize()
    assert (O.cpu() == 3.0).all() and (L.cpu() == 5.0).all()


def test_explicit_stream(sattn, dev):
    import torch
    x = make_inputs(257, 8, 2, seed=11)
    s = torch.cuda.Stream(device=dev)
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        O, L = sattn.fwd(q, k, vt, x.c)
    s.synchronize()
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64), Or, Lr,
                 "side stream")
