"""Parity of the eight-wave forward kernel (the one the benchmark times) with
the float64 oracle, over whole outputs.

Every shape here is one that the library sends to its eight-wave kernel:
enough query-block pairs that every compute unit gets an eight-wave workgroup
(`eight_wave` restates that host-side rule, and each test asserts it first).
The two large synthetic workloads are compared element by element in full;
around them, canaries before and after O and L, bitwise determinism, bitwise
causality, a side stream, V given as rows, K and V followed by binary16 NaN
(reads must stay inside the planes), and the largest admitted sequence length
for one head, where the per-head buffer offsets peak.

Tolerances (stated for the attention forward): max |O - O_ref| <= 4e-3 and
max |L - L_ref| <= 2e-4 (base-2 units), element by element.
"""
import numpy as np
import pytest

from causal_attention_forward_amd.inputs import WORKLOADS, make_inputs, make_workload
from oracle import attention_ref, attention_rows_ref
from parity_util import TOL_L, TOL_O, assert_close, note, run

pytestmark = pytest.mark.gpu

N_CUS = 256


def eight_wave(T, Hq, Hkv):
    """The library's routing rule: 32-row query blocks are paired (heavy,
    light); a workgroup holds GW heads of a group times 8/GW pair slots, and
    the eight-wave kernel runs when that grid covers every compute unit."""
    G = Hq // Hkv
    gw = 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    pairs = ((T + 31) // 32 + 1) // 2
    rs = 8 // gw
    return ((pairs + rs - 1) // rs) * Hkv * (G // gw) >= N_CUS


def to_dev(dev, x):
    import torch
    return (torch.from_numpy(x.Q).to(dev), torch.from_numpy(x.K).to(dev),
            torch.from_numpy(x.Vt).to(dev))


@pytest.mark.parametrize("idx", [3, 4])
def test_workload_full_main(sattn, dev, idx):
    w = WORKLOADS[idx]
    assert eight_wave(w.T, w.Hq, w.Hkv)
    note(f"workload {idx} ({w.name}) full compare, eight-wave kernel")
    x = make_workload(idx)
    O, L = run(sattn, dev, x)
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O, L, Or, Lr, w.name)


@pytest.mark.parametrize("T,Hq,Hkv", [(1024, 128, 32), (4000, 32, 8), (4095, 32, 8)])
def test_guard_bands_main(sattn, dev, T, Hq, Hkv):
    """O and L written exactly inside their extents by the eight-wave kernel's
    whole-row O stores (canaries before and after both stay intact), and the
    whole output within tolerance.  T=4000 has an odd number of 32-row blocks
    (its middle block has no light partner); T=4095 is ragged and takes the
    element-wise V^T path for its last tile."""
    import torch
    assert eight_wave(T, Hq, Hkv)
    note(f"guard bands T={T} Hq={Hq} Hkv={Hkv}")
    x = make_inputs(T, Hq, Hkv, seed=31 + T)
    q, k, vt = to_dev(dev, x)
    pad = 8192
    ob = torch.full((pad + T * Hq * 64 + pad,), 12345.0, dtype=torch.float16, device=dev)
    lb = torch.full((pad + Hq * T + pad,), -777.0, dtype=torch.float32, device=dev)
    O = ob[pad:pad + T * Hq * 64].view(T, Hq * 64)
    L = lb[pad:pad + Hq * T].view(Hq, T)
    sattn.fwd(q, k, vt, x.c, out=O, lse=L)
    torch.cuda.synchronize()
    obh, lbh = ob.cpu().numpy(), lb.cpu().numpy()
    assert (obh[:pad] == np.float16(12345.0)).all() and (obh[-pad:] == np.float16(12345.0)).all()
    assert (lbh[:pad] == -777.0).all() and (lbh[-pad:] == -777.0).all()
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64), Or, Lr,
                 f"guarded T={T} Hq={Hq} Hkv={Hkv}")


def test_deterministic_main(sattn, dev):
    assert eight_wave(4096, 32, 8)
    note("bitwise determinism, T=4096 Hq=32 Hkv=8")
    x = make_workload(3)
    O1, L1 = run(sattn, dev, x)
    O2, L2 = run(sattn, dev, x)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_causality_bitwise_main(sattn, dev):
    """Changing keys and values after row i0 leaves rows 0..i0 bit-identical.
    i0 ends a 64-key tile, so no wave holds rows on both sides of it (a
    wave's rescale decision is taken for all its rows at once)."""
    T, Hq, Hkv = 1024, 128, 32
    assert eight_wave(T, Hq, Hkv)
    note(f"bitwise causality T={T} Hq={Hq} Hkv={Hkv}")
    x = make_inputs(T, Hq, Hkv, seed=32)
    O1, L1 = run(sattn, dev, x)
    i0 = 511
    rng = np.random.default_rng(4)
    x.K[:, i0 + 1:] = rng.standard_normal(x.K[:, i0 + 1:].shape).astype(np.float16)
    x.Vt[:, :, i0 + 1:] = rng.standard_normal(x.Vt[:, :, i0 + 1:].shape).astype(np.float16)
    O2, L2 = run(sattn, dev, x)
    assert np.array_equal(O1[:i0 + 1], O2[:i0 + 1]) and np.array_equal(L1[:, :i0 + 1], L2[:, :i0 + 1])
    assert not np.array_equal(O1[i0 + 1:], O2[i0 + 1:])


def test_side_stream_main(sattn, dev):
    import torch
    T, Hq, Hkv = 1024, 128, 32
    assert eight_wave(T, Hq, Hkv)
    note(f"side stream T={T} Hq={Hq} Hkv={Hkv}")
    x = make_inputs(T, Hq, Hkv, seed=33)
    s = torch.cuda.Stream(device=dev)
    q, k, vt = to_dev(dev, x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        O, L = sattn.fwd(q, k, vt, x.c)
    s.synchronize()
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64), Or, Lr,
                 "side stream, eight-wave")


def test_vrows_full_main(sattn, dev):
    """sattn_fwd_vrows at the headline workload: the whole output against the
    oracle, and bit-identical to sattn_fwd on the same values."""
    assert eight_wave(4096, 32, 8)
    note("V rows, T=4096 Hq=32 Hkv=8, full compare")
    x = make_workload(3)
    q, k, vt = to_dev(dev, x)
    v = vt.transpose(1, 2).contiguous()
    O, L = sattn.fwd_vrows(q, k, v, x.c)
    O2, L2 = sattn.fwd(q, k, vt, x.c)
    import torch
    torch.cuda.synchronize()
    O, L = O.cpu().numpy(), L.cpu().numpy()
    assert np.array_equal(O, O2.cpu().numpy()) and np.array_equal(L, L2.cpu().numpy())
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O.astype(np.float64), L.astype(np.float64), Or, Lr, "V rows T=4096")


@pytest.mark.parametrize("T,vrows", [(4095, False), (4095, True), (4000, False), (4000, True)])
def test_nan_after_planes(sattn, dev, T, vrows):
    """K and V (or V^T) at the start of larger buffers whose tails hold
    binary16 NaN: rows past T of the ragged last tile, and tiles past the
    last, must read as zeros through the buffer range checks, never from the
    memory after the planes (V rows times P = 0 would otherwise turn NaN into
    O).  Every read stays inside the allocations.  T=4095 takes the
    element-wise V^T path for its last tile, T=4000 the 16-byte one."""
    import torch
    Hq, Hkv = 32, 8
    assert eight_wave(T, Hq, Hkv)
    note(f"NaN after the K/V planes, T={T} Hq={Hq} Hkv={Hkv} vrows={vrows}")
    x = make_inputs(T, Hq, Hkv, seed=34)
    q = torch.from_numpy(x.Q).to(dev)
    tail = 1 << 20
    n = Hkv * T * 64
    kb = torch.full((n + tail,), float("nan"), dtype=torch.float16, device=dev)
    vb = torch.full((n + tail,), float("nan"), dtype=torch.float16, device=dev)
    kb[:n].copy_(torch.from_numpy(x.K).reshape(-1).to(dev))
    if vrows:
        vb[:n].copy_(torch.from_numpy(np.ascontiguousarray(x.Vt.transpose(0, 2, 1))).reshape(-1).to(dev))
        O, L = sattn.fwd_vrows(q, kb[:n].view(Hkv, T, 64), vb[:n].view(Hkv, T, 64), x.c)
    else:
        vb[:n].copy_(torch.from_numpy(x.Vt).reshape(-1).to(dev))
        O, L = sattn.fwd(q, kb[:n].view(Hkv, T, 64), vb[:n].view(Hkv, 64, T), x.c)
    torch.cuda.synchronize()
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64), Or, Lr,
                 f"NaN tails, vrows={vrows}")


@pytest.mark.timeout(600)
def test_longest_admitted_head(sattn, dev):
    """Hq = Hkv = 1 at T = 16,777,215, the largest T the admission rule
    (Hq * 64 * T * 4 <= 2^32 - 1) allows: the per-head planes hold 2^31 - 128
    bytes, so the V^T row offsets and the K tile offsets of the last tiles
    are the largest any call makes.  Inputs: seeded rows of a base of
    P = 131,101 tokens (not a power of two, so an offset error by a power of
    two reads different data) repeated along the tokens, and Q rows taken
    from the base with stride 7.  Sampled rows (most of them near the end,
    where every tile of the plane is visited) against the float64 oracle;
    every L finite and every row a convex combination of V."""
    import torch
    T = 16_777_215
    assert 64 * T * 4 <= 2 ** 32 - 1 < 64 * (T + 1) * 4
    assert eight_wave(T, 1, 1)
    P = 131_101
    note(f"longest admitted head T={T}: building inputs")
    base = make_inputs(P, 1, 1, seed=35)
    reps = -(-T // P)
    qi = (np.arange(T, dtype=np.int64) * 7) % P
    Qh = base.Q[0][qi][None]                                       # [1][T][64]
    Kh = np.tile(base.K[0], (reps, 1))[:T][None]                   # [1][T][64]
    Vth = np.ascontiguousarray(np.tile(base.Vt[0], (1, reps))[:, :T][None])  # [1][64][T]
    q = torch.from_numpy(Qh).to(dev)
    k = torch.from_numpy(Kh).to(dev)
    vt = torch.from_numpy(Vth).to(dev)
    note("  running the forward (about a minute of GPU time)")
    O, L = sattn.fwd(q, k, vt, base.c)
    torch.cuda.synchronize()
    note("  forward done")
    Lh = L.cpu().numpy()
    assert np.isfinite(Lh).all()
    Oh = O.cpu().numpy()
    assert np.isfinite(Oh).all()
    bound = np.abs(base.Vt[0].astype(np.float64)).max(axis=1) * (1 + 2e-3) + 1e-3
    assert (np.abs(Oh.astype(np.float64)) <= bound[None, :]).all()
    del Oh
    rows = [0, 1, 63, 64, P - 1, P, T // 2, T - 4096, T - 1000, T - 65, T - 64, T - 63, T - 2, T - 1]
    note(f"  oracle on {len(rows)} rows")
    Or, Lr = attention_rows_ref(Qh, Kh, Vth, base.c, 0, rows, key_chunk=1 << 20)
    Og = O[rows].cpu().numpy().astype(np.float64)
    eo = float(np.abs(Og - Or).max())
    el = float(np.abs(Lh[0, rows].astype(np.float64) - Lr).max())
    note(f"  T={T}: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_L


@pytest.mark.parametrize("T,Hq,Hkv", [(4096, 32, 8), (4096, 32, 16), (4000, 64, 32)])
def test_gqa_replication_bitwise(sattn, dev, T, Hq, Hkv):
    """K and V^T repeated per query head (Hkv = Hq) give bit-identical O and L:
    a row's arithmetic does not depend on how many heads share its K/V, so the
    eight-wave kernel's group widths 4 and 2 are checked against its
    one-head-per-group build at full size."""
    import torch
    assert eight_wave(T, Hq, Hkv) and eight_wave(T, Hq, Hq)
    note(f"GQA replication T={T} Hq={Hq} Hkv={Hkv} vs Hkv={Hq}")
    x = make_inputs(T, Hq, Hkv, seed=41)
    q, k, vt = to_dev(dev, x)
    O1, L1 = sattn.fwd(q, k, vt, x.c)
    G = Hq // Hkv
    O2, L2 = sattn.fwd(q, k.repeat_interleave(G, 0).contiguous(),
                       vt.repeat_interleave(G, 0).contiguous(), x.c)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
