"""The entry points captured in a HIP graph and replayed (a serving loop, or a
model layer wired as a captured graph, calls them this way).

Each case captures one call with its outputs preallocated, then replays the
graph three times.  Before every replay the outputs are filled with NaN and
other eager work runs on the device (the library's own eager calls on other
buffers, torch fills); each replay must reproduce the eager call's outputs bit
for bit.  Before the last replay the inputs are overwritten in place with a
second input set, so the replay must read the live inputs: it is compared with
an eager call on that second set.  Covered: the eight-wave forward, the
split-key forward (LDS-staged, register-staged, and T % 8 != 0), V given as
rows, the backward (split launches with the grouped reduction, and the
eight-wave launches), the key launch with the library's static workspace, and
the materialised path's three launches.
The library allocates nothing and records no memset, so a capture holds only
its kernels.  One forward replay is also checked against the float64 oracle.
"""
import numpy as np
import pytest

from causal_attention_forward_amd.inputs import make_inputs, make_output_gradient
from oracle import attention_ref
from parity_util import TOL_L, TOL_O, note

pytestmark = pytest.mark.gpu

S = 0.125


def _capture(torch, fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(torch, g, outs, expect, between, swap_inputs, expect_swapped):
    """Three replays: NaN-filled outputs, eager work in between, bitwise
    equality with the eager outputs; the last after swap_inputs()."""
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        between()
        if r == 2:
            swap_inputs()
            expect = expect_swapped()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, expect):
            assert torch.equal(o, e), f"replay {r} differs from the eager call"


FWD_CASES = [
    (2048, 64, 16, "eight-wave"),
    (1024, 8, 8, "split-key, LDS-staged"),
    (1000, 16, 4, "split-key, register-staged"),
    (999, 4, 2, "split-key, T % 8 != 0"),
]


@pytest.mark.parametrize("T,Hq,Hkv,kind", FWD_CASES)
@pytest.mark.parametrize("vrows", [False, True])
def test_forward_graph_replay(sattn, dev, T, Hq, Hkv, kind, vrows):
    import torch
    note(f"graph replay forward T={T} Hq={Hq} Hkv={Hkv} ({kind}) vrows={vrows}")
    x = make_inputs(T, Hq, Hkv, seed=71)
    y = make_inputs(T, Hq, Hkv, seed=72)
    q, k, vt = (torch.from_numpy(a).to(dev) for a in (x.Q, x.K, x.Vt))
    v = vt.transpose(1, 2).contiguous()  # V rows [Hkv][T][64]
    third = v if vrows else vt
    call = sattn.fwd_vrows if vrows else sattn.fwd
    O = torch.empty((T, Hq * 64), dtype=torch.float16, device=dev)
    L = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    Oe, Le = call(q, k, third, x.c)
    g = _capture(torch, lambda: call(q, k, third, x.c, out=O, lse=L))
    # eager work between replays: the library on other buffers, torch fills
    q2, k2 = (torch.from_numpy(a).to(dev) for a in (y.Q, y.K))
    scratch_O = torch.empty_like(O)
    scratch_L = torch.empty_like(L)

    def between():
        call(q2, k2, third, x.c, out=scratch_O, lse=scratch_L)
        scratch_O.fill_(0)

    def swap():
        q.copy_(torch.from_numpy(y.Q))
        k.copy_(torch.from_numpy(y.K))

    def swapped():
        return call(torch.from_numpy(y.Q).to(dev), torch.from_numpy(y.K).to(dev), third, x.c)

    _replays(torch, g, [O, L], [Oe, Le], between, swap, swapped)
    if T <= 1024:
        Or, Lr = attention_ref(y.Q, y.K, x.Vt, x.c)
        eo = float(np.abs(O.cpu().numpy().astype(np.float64) - Or).max())
        el = float(np.abs(L.cpu().numpy().astype(np.float64) - Lr).max())
        note(f"  last replay against the oracle: max|dO|={eo:.3e} max|dL|={el:.3e}")
        assert eo <= TOL_O and el <= TOL_L


BWD_CASES = [
    (1000, 16, 4, "split launches + grouped reduction"),
    (2048, 64, 16, "eight-wave launches + grouped reduction"),
]


@pytest.mark.parametrize("T,Hq,Hkv,kind", BWD_CASES)
def test_backward_graph_replay(sattn, dev, T, Hq, Hkv, kind):
    import torch
    note(f"graph replay backward T={T} Hq={Hq} Hkv={Hkv} ({kind})")
    x = make_inputs(T, Hq, Hkv, seed=73)
    q, k, vt = (torch.from_numpy(a).to(dev) for a in (x.Q, x.K, x.Vt))
    do = torch.from_numpy(make_output_gradient(T, Hq, 73)).to(dev)
    do2 = torch.from_numpy(make_output_gradient(T, Hq, 74)).to(dev)
    O, L = sattn.fwd(q, k, vt, x.c)
    f32 = dict(dtype=torch.float32, device=dev)
    outs = [torch.empty((Hq, T, 64), **f32), torch.empty((Hkv, T, 64), **f32),
            torch.empty((Hkv, 64, T), **f32), torch.empty((Hq, T), **f32)]
    ws = torch.empty(max(sattn.sattn_bwd_workspace_bytes(T, Hq, Hkv), 16), dtype=torch.uint8,
                     device=dev)
    expect = [t.clone() for t in sattn.bwd(q, k, vt, O, do, L, x.c, S, workspace=ws)]
    g = _capture(torch, lambda: sattn.bwd(q, k, vt, O, do, L, x.c, S, dq=outs[0], dk=outs[1],
                                          dvt=outs[2], D=outs[3], workspace=ws))
    ws2 = torch.empty_like(ws)
    junk = [torch.empty_like(t) for t in outs]

    def between():
        sattn.bwd(q, k, vt, O, do2, L, x.c, S, dq=junk[0], dk=junk[1], dvt=junk[2], D=junk[3],
                  workspace=ws2)
        junk[0].fill_(0)

    def swap():
        do.copy_(do2)

    def swapped():
        return [t.clone() for t in sattn.bwd(q, k, vt, O, do2, L, x.c, S, workspace=ws2)]

    _replays(torch, g, outs, expect, between, swap, swapped)


def test_noalloc_key_launch_graph_replay(sattn, dev):
    """sattn_bwd_key_noalloc captured: its static region is the workspace of
    every replay, with an eager call of it on another problem in between."""
    import torch
    T, Hq, Hkv = 1000, 16, 4
    note(f"graph replay of the no-alloc key launch T={T} Hq={Hq} Hkv={Hkv}")
    x = make_inputs(T, Hq, Hkv, seed=75)
    q, k, vt = (torch.from_numpy(a).to(dev) for a in (x.Q, x.K, x.Vt))
    do = torch.from_numpy(make_output_gradient(T, Hq, 75)).to(dev)
    O, L = sattn.fwd(q, k, vt, x.c)
    f32 = dict(dtype=torch.float32, device=dev)
    _, _, _, D = sattn.bwd(q, k, vt, O, do, L, x.c, S)
    p = lambda t: t.data_ptr()  # noqa: E731
    dK, dVt = torch.empty((Hkv, T, 64), **f32), torch.empty((Hkv, 64, T), **f32)

    def key(dk, dvt, stream):
        assert sattn.sattn_bwd_key_noalloc(p(q), p(k), p(vt), p(do), p(L), p(D), p(dk), p(dvt),
                                           x.c, S, T, Hq, Hkv, stream) == sattn.SATTN_OK

    eK, eVt = torch.empty_like(dK), torch.empty_like(dVt)
    key(eK, eVt, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    g = _capture(torch, lambda: key(dK, dVt, torch.cuda.current_stream().cuda_stream))
    # another problem through the same static region between replays
    y = make_inputs(257, 6, 2, seed=76)
    q2, k2, vt2 = (torch.from_numpy(a).to(dev) for a in (y.Q, y.K, y.Vt))
    do2 = torch.from_numpy(make_output_gradient(257, 6, 76)).to(dev)
    O2, L2 = sattn.fwd(q2, k2, vt2, y.c)
    _, _, _, D2 = sattn.bwd(q2, k2, vt2, O2, do2, L2, y.c, S)
    jK, jVt = torch.empty((2, 257, 64), **f32), torch.empty((2, 64, 257), **f32)

    def between():
        assert sattn.sattn_bwd_key_noalloc(p(q2), p(k2), p(vt2), p(do2), p(L2), p(D2), p(jK),
                                           p(jVt), y.c, S, 257, 6, 2,
                                           torch.cuda.current_stream().cuda_stream) == sattn.SATTN_OK

    _replays(torch, g, [dK, dVt], [eK, eVt], between, lambda: None, lambda: [eK, eVt])


MAT_CASES = [(1000, 16, 4), (257, 6, 2)]


@pytest.mark.parametrize("T,Hq,Hkv", MAT_CASES)
def test_materialised_graph_replay(sattn, dev, T, Hq, Hkv):
    """sattn_mat_fwd captured (scores, softmax and P.V launches): the planes and
    O, L of every replay equal the eager call's; the last after new Q and K."""
    import torch
    note(f"graph replay materialised T={T} Hq={Hq} Hkv={Hkv}")
    x = make_inputs(T, Hq, Hkv, seed=77)
    y = make_inputs(T, Hq, Hkv, seed=78)
    q, k, vt = (torch.from_numpy(a).to(dev) for a in (x.Q, x.K, x.Vt))
    O = torch.empty((T, Hq * 64), dtype=torch.float16, device=dev)
    L = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    S = torch.zeros((Hq, T, T), dtype=torch.float32, device=dev)
    P = torch.zeros((Hq, T, T), dtype=torch.float16, device=dev)
    Oe, Le, Se, Pe = (t.clone() for t in sattn.mat_fwd(q, k, vt, x.c, scores=S, probs=P))
    g = _capture(torch, lambda: sattn.mat_fwd(q, k, vt, x.c, scores=S, probs=P, out=O, lse=L))
    q2, k2 = (torch.from_numpy(a).to(dev) for a in (y.Q, y.K))
    jO, jL = torch.empty_like(O), torch.empty_like(L)
    jS, jP = torch.zeros_like(S), torch.zeros_like(P)
    tri = torch.tril(torch.ones((T, T), dtype=torch.bool, device=dev))

    def between():
        sattn.mat_fwd(q2, k2, vt, x.c, scores=jS, probs=jP, out=jO, lse=jL)
        jO.fill_(0)

    def swap():
        q.copy_(torch.from_numpy(y.Q))
        k.copy_(torch.from_numpy(y.K))

    def swapped():
        S2, P2 = torch.zeros_like(S), torch.zeros_like(P)
        r = sattn.mat_fwd(torch.from_numpy(y.Q).to(dev), torch.from_numpy(y.K).to(dev), vt, x.c,
                          scores=S2, probs=P2)
        return [r[0], r[1]]

    # the planes keep whatever is above the diagonal, so only O and L are NaN-filled
    # between replays and the planes are compared on and below the diagonal
    for r in range(3):
        O.fill_(float("nan"))
        L.fill_(float("nan"))
        S.masked_fill_(tri, float("nan"))
        P.masked_fill_(tri, float("nan"))
        between()
        if r == 2:
            swap()
            expect = swapped()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if r < 2:
            assert torch.equal(O, Oe) and torch.equal(L, Le), f"replay {r} differs from the eager call"
            assert torch.equal(S[:, tri], Se[:, tri]) and torch.equal(P[:, tri], Pe[:, tri])
        else:
            assert torch.equal(O, expect[0]) and torch.equal(L, expect[1])
