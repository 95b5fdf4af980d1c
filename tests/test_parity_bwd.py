"""Parity of the HIP backward with the float64 backward oracle, through the C
ABI, element by element within bounds derived from the HIP path's arithmetic
(binary16 rounding of P and dS, binary32 sums; see bwd_util).

Small and medium shapes are compared in full (every element of dQ, dK, dV and
D); the full-size shapes on sampled query rows of every head and sampled keys
of every K/V head, each computed one by one by the oracle.
"""
import numpy as np
import pytest

from bwd_util import Case, check_within, key_rows_expected, query_rows_expected, run_bwd
from parity_util import note, sample_rows

pytestmark = pytest.mark.gpu

# (T, Hq, Hkv, seed, generator options): tiny and degenerate shapes, ragged
# tails, T not a multiple of 8 (scalar V^T staging), odd groups, the small
# and medium forward workloads' shapes and value distributions (these take
# the split launches: 32-row blocks, tiles dealt over four waves)
FULL = [
    (1, 1, 1, 51, {}),
    (2, 2, 1, 52, {}),
    (64, 2, 2, 53, {}),
    (77, 3, 1, 54, {}),
    (128, 1, 1, 0, {}),
    (200, 4, 2, 55, {}),
    (333, 6, 2, 56, {"peaked_fraction": 0.02}),
    (257, 2, 2, 57, {"qk_std": 1.5}),
    (1000, 16, 4, 2, {"peaked_fraction": 0.01}),
    (1024, 8, 8, 1, {"qk_std": 0.5, "v_std": 0.5}),
    # a split grid that fits the chip at once (LDS-staged tiles on both sides)
    # with a ragged last tile and groups of four
    (1000, 8, 2, 58, {"peaked_fraction": 0.01}),
    # grids large enough for heavy/light block pairing: four-wave workgroups
    # with an odd block count (the middle block pairs with itself) and a
    # non-multiple-of-8 tail, and with an even count; eight-wave workgroups
    # with an odd count, and with a non-multiple-of-8 tail
    (300, 128, 16, 61, {}),
    (512, 128, 16, 63, {}),
    (520, 128, 64, 62, {}),
    (777, 128, 64, 64, {}),
    # one 128-row block over many heads: four-wave workgroups, unpaired
    (100, 512, 8, 65, {}),
]


@pytest.mark.parametrize("T,Hq,Hkv,seed,kw", FULL,
                         ids=[f"T{t}_Hq{a}_Hkv{b}" for t, a, b, _, _ in FULL])
def test_backward_full(sattn, dev, T, Hq, Hkv, seed, kw):
    note(f"backward full compare T={T} Hq={Hq} Hkv={Hkv} seed={seed} {kw}")
    case = Case(T, Hq, Hkv, seed, **kw)
    dQ, dK, dVt, D = run_bwd(sattn, dev, case)
    rows = list(range(T))
    for h in range(Hq):
        want, tol, Dw, Dtol = query_rows_expected(case, h, rows)
        check_within(dQ[h], want, tol, f"dQ head {h}", note)
        check_within(D[h], Dw, Dtol, f"D head {h}", note)
    for kv in range(Hkv):
        wk, tk, wv, tv = key_rows_expected(case, kv, rows)
        check_within(dK[kv], wk, tk, f"dK head {kv}", note)
        check_within(dVt[kv].T, wv, tv, f"dV head {kv}", note)


SAMPLED = [
    (4096, 32, 8, 3, {}),
    (4095, 8, 2, 58, {}),
]


@pytest.mark.parametrize("T,Hq,Hkv,seed,kw", SAMPLED,
                         ids=[f"T{t}_Hq{a}_Hkv{b}" for t, a, b, _, _ in SAMPLED])
def test_backward_sampled(sattn, dev, T, Hq, Hkv, seed, kw):
    note(f"backward sampled compare T={T} Hq={Hq} Hkv={Hkv} seed={seed}")
    case = Case(T, Hq, Hkv, seed, **kw)
    dQ, dK, dVt, D = run_bwd(sattn, dev, case)
    assert all(np.isfinite(a).all() for a in (dQ, dK, dVt, D))
    rng = np.random.default_rng(seed)
    for h in range(Hq):
        rows = sample_rows(T, rng, extra=4)
        want, tol, Dw, Dtol = query_rows_expected(case, h, rows)
        check_within(dQ[h, rows], want, tol, f"dQ head {h}", note)
        check_within(D[h, rows], Dw, Dtol, f"D head {h}", note)
    for kv in range(Hkv):
        keys = sample_rows(T, rng, extra=4)
        wk, tk, wv, tv = key_rows_expected(case, kv, keys)
        check_within(dK[kv, keys], wk, tk, f"dK head {kv}", note)
        check_within(dVt[kv][:, keys].T, wv, tv, f"dV head {kv}", note)


def test_backward_deterministic_and_split_launches(sattn, dev):
    """The same inputs give the same bits twice, and the query launch followed
    by the key launch (separate entry points) gives the combined result."""
    import torch
    case = Case(700, 8, 2, 59)
    a = run_bwd(sattn, dev, case)
    b = run_bwd(sattn, dev, case)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    t = lambda arr: torch.from_numpy(np.ascontiguousarray(arr)).to(dev)  # noqa: E731
    x = case.x
    q, k, vt, o, do, L = t(x.Q), t(x.K), t(x.Vt), t(case.O), t(case.dO), t(case.L)
    T, Hq, Hkv = case.T, case.Hq, case.Hkv
    dQ = torch.empty((Hq, T, 64), dtype=torch.float32, device=dev)
    D = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    dK = torch.empty((Hkv, T, 64), dtype=torch.float32, device=dev)
    dVt = torch.empty((Hkv, 64, T), dtype=torch.float32, device=dev)
    need = sattn.sattn_bwd_workspace_bytes(T, Hq, Hkv)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    assert sattn.sattn_bwd_query(q.data_ptr(), k.data_ptr(), vt.data_ptr(), o.data_ptr(),
                                 do.data_ptr(), L.data_ptr(), dQ.data_ptr(), D.data_ptr(),
                                 case.c, case.s, T, Hq, Hkv, stream) == sattn.SATTN_OK
    assert sattn.sattn_bwd_key(q.data_ptr(), k.data_ptr(), vt.data_ptr(), do.data_ptr(),
                               L.data_ptr(), D.data_ptr(), dK.data_ptr(), dVt.data_ptr(),
                               ws.data_ptr(), need, case.c, case.s, T, Hq, Hkv,
                               stream) == sattn.SATTN_OK
    torch.cuda.synchronize()
    for got, want in zip((dQ, dK, dVt, D), a):
        assert np.array_equal(got.cpu().numpy().astype(np.float64), want)


def test_backward_rejects_small_workspace(sattn, dev):
    import torch
    case = Case(128, 4, 2, 60)
    x = case.x
    t = lambda arr: torch.from_numpy(np.ascontiguousarray(arr)).to(dev)  # noqa: E731
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(sattn.SattnError) as e:
        sattn.bwd(t(x.Q), t(x.K), t(x.Vt), t(case.O), t(case.dO), t(case.L), case.c, case.s,
                  workspace=small)
    assert e.value.status == sattn.SATTN_ERR_WORKSPACE
