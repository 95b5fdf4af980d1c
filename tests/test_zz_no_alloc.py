"""sattn_bwd_key_noalloc (the key launch with the library's static workspace)
against sattn_bwd_key with a caller workspace, through the C ABI.

Calls in a row with decreasing sizes: the first needs exactly the static
region (T=4096, Hq=32, Hkv=8: 64 MiB), the next ones less, ragged T, a
split-launch shape, and Hq = Hkv (no workspace at all), so each call runs on
what the previous one left in the region.  The two entry points run the same
kernels in the same order, so dK and dV^T must agree bit for bit; the outputs
start as NaN so a plane left unwritten shows.  A problem one token larger
than the region allows is refused with SATTN_ERR_SCRATCH and launches
nothing.
"""
import numpy as np
import pytest

from causal_attention_forward_amd.inputs import make_inputs, make_output_gradient

pytestmark = pytest.mark.gpu

CASES = [(4096, 32, 8), (1000, 16, 4), (257, 6, 2), (200, 4, 4)]
S = 0.125


def _run_pair(sattn, dev, T, Hq, Hkv, seed):
    import torch
    x = make_inputs(T, Hq, Hkv, seed=seed)
    q, k, vt = (torch.from_numpy(a).to(dev) for a in (x.Q, x.K, x.Vt))
    do = torch.from_numpy(make_output_gradient(T, Hq, seed)).to(dev)
    O, L = sattn.fwd(q, k, vt, x.c)
    f32 = dict(dtype=torch.float32, device=dev)
    dQ, D = torch.empty((Hq, T, 64), **f32), torch.empty((Hq, T), **f32)
    p = lambda t: t.data_ptr()  # noqa: E731
    assert sattn.sattn_bwd_query(p(q), p(k), p(vt), p(O), p(do), p(L), p(dQ), p(D), x.c, S, T, Hq,
                                 Hkv, None) == sattn.SATTN_OK
    need = sattn.sattn_bwd_workspace_bytes(T, Hq, Hkv)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    dK_ref = torch.full((Hkv, T, 64), float("nan"), **f32)
    dVt_ref = torch.full((Hkv, 64, T), float("nan"), **f32)
    assert sattn.sattn_bwd_key(p(q), p(k), p(vt), p(do), p(L), p(D), p(dK_ref), p(dVt_ref),
                               p(ws) if need else None, need, x.c, S, T, Hq, Hkv,
                               None) == sattn.SATTN_OK
    dK = torch.full((Hkv, T, 64), float("nan"), **f32)
    dVt = torch.full((Hkv, 64, T), float("nan"), **f32)
    torch.cuda.synchronize()
    assert sattn.sattn_bwd_key_noalloc(p(q), p(k), p(vt), p(do), p(L), p(D), p(dK), p(dVt), x.c,
                                       S, T, Hq, Hkv, None) == sattn.SATTN_OK
    torch.cuda.synchronize()
    a, b = dK.cpu().numpy(), dK_ref.cpu().numpy()
    c, d = dVt.cpu().numpy(), dVt_ref.cpu().numpy()
    assert np.isfinite(b).all() and np.isfinite(d).all()
    assert np.array_equal(a, b), f"dK differs at T={T} Hq={Hq} Hkv={Hkv}"
    assert np.array_equal(c, d), f"dVt differs at T={T} Hq={Hq} Hkv={Hkv}"
    return need


def test_noalloc_key_launch_matches_workspace_entry(sattn, dev):
    needs = []
    for i, (T, Hq, Hkv) in enumerate(CASES):
        print(f"no-alloc key launch T={T} Hq={Hq} Hkv={Hkv}", flush=True)
        needs.append(_run_pair(sattn, dev, T, Hq, Hkv, seed=50 + i))
    assert needs[0] == sattn.BWD_NOALLOC_MAX_BYTES
    assert needs == sorted(needs, reverse=True) and needs[-1] == 0


def test_noalloc_refuses_more_than_its_region(sattn, dev):
    import torch
    T, Hq, Hkv = 4097, 32, 8
    assert sattn.sattn_bwd_workspace_bytes(T, Hq, Hkv) > sattn.BWD_NOALLOC_MAX_BYTES
    f16 = dict(dtype=torch.float16, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    q, do = torch.zeros((Hq, T, 64), **f16), torch.zeros((T, Hq * 64), **f16)
    k, vt = torch.zeros((Hkv, T, 64), **f16), torch.zeros((Hkv, 64, T), **f16)
    L, D = torch.zeros((Hq, T), **f32), torch.zeros((Hq, T), **f32)
    dK = torch.full((Hkv, T, 64), 7.0, **f32)
    dVt = torch.full((Hkv, 64, T), 7.0, **f32)
    p = lambda t: t.data_ptr()  # noqa: E731
    st = sattn.sattn_bwd_key_noalloc(p(q), p(k), p(vt), p(do), p(L), p(D), p(dK), p(dVt), 0.18, S,
                                     T, Hq, Hkv, None)
    assert st == sattn.SATTN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (dK == 7.0).all() and (dVt == 7.0).all()
