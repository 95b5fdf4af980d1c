"""Parity on inputs built to drive the kernels' less common paths, on both
kernels (the eight-wave main kernel when its grid fills every CU, the
split-key kernel otherwise).

* Rising scores: keys carry a ramp along the sequence, so a row's running
  maximum grows by several base-2 units per 64-key tile and the reference
  must be raised again and again (the exact power-of-two rescale).
* Score spikes: two keys whose scores exceed everything before them by far
  more than 128 base-2 units, so 2^(t - m) overflows binary32 and the tile's
  scores are formed again and the reference taken from their maximum; the
  second spike falls inside the diagonal (masked) tile of some rows.
* Shapes whose grid selects the eight-wave workgroup with T % 8 != 0, with
  two or one query heads per K/V head, and with an odd number of query blocks.
Full oracle comparison where it runs in seconds, sampled rows otherwise.
"""
import numpy as np
import pytest

from causal_attention_forward_amd.inputs import make_inputs
from oracle import attention_ref, attention_rows_ref
from parity_util import TOL_L, TOL_O, assert_close, note, run, sample_rows

pytestmark = pytest.mark.gpu

# (T, Hq, Hkv): the first two take the split-key kernel (LDS-staged, lazy
# reference), the third the main kernel
PATH_SHAPES = [(1000, 8, 2), (2048, 4, 4), (4096, 32, 8)]


def rising(T, Hq, Hkv, seed):
    """Positive queries and a ramp of 6 * k / T on every element of key k."""
    x = make_inputs(T, Hq, Hkv, seed=seed)
    x.Q[:] = (np.abs(x.Q.astype(np.float32)) + 0.25).astype(np.float16)
    ramp = (6.0 * np.arange(T, dtype=np.float32) / T)[None, :, None]
    x.K[:] = (x.K.astype(np.float32) + ramp).astype(np.float16)
    return x


def spiked(T, Hq, Hkv, seed):
    """Positive queries; key T/3 + 5 set to 24 and key 2T/3 + 40 to 40 on
    every element (scores of about 2000 and 3300, i.e. jumps of hundreds of
    base-2 units over the running maximum)."""
    x = make_inputs(T, Hq, Hkv, seed=seed)
    x.Q[:] = (np.abs(x.Q.astype(np.float32)) + 0.5).astype(np.float16)
    k1, k2 = T // 3 + 5, 2 * T // 3 + 40
    x.K[:, k1, :] = np.float16(24.0)
    x.K[:, k2, :] = np.float16(40.0)
    return x, (k1, k2)


def compare(sattn, dev, x, what, extra_rows=()):
    O, L = run(sattn, dev, x)
    if x.T * x.Hq <= 1000 * 8:
        Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
        assert_close(O, L, Or, Lr, what)
        return O, L
    rng = np.random.default_rng(x.T + x.Hq)
    worst_o = worst_l = 0.0
    for h in range(x.Hq):
        rows = sorted(set(sample_rows(x.T, rng, extra=8)) | {r for r in extra_rows if 0 <= r < x.T})
        Or, Lr = attention_rows_ref(x.Q, x.K, x.Vt, x.c, h, rows)
        assert np.isfinite(O[rows]).all() and np.isfinite(L[h, rows]).all()
        worst_o = max(worst_o, float(np.abs(O[rows, h * 64:(h + 1) * 64] - Or).max()))
        worst_l = max(worst_l, float(np.abs(L[h, rows] - Lr).max()))
    note(f"  {what} (sampled rows): max|dO|={worst_o:.3e} max|dL|={worst_l:.3e}")
    assert worst_o <= TOL_O and worst_l <= TOL_L
    return O, L


@pytest.mark.parametrize("shape", PATH_SHAPES)
def test_rising_scores(sattn, dev, shape):
    T, hq, hkv = shape
    note(f"rising scores T={T} Hq={hq} Hkv={hkv}")
    x = rising(T, hq, hkv, seed=21)
    compare(sattn, dev, x, f"rising T={T}")


@pytest.mark.parametrize("shape", PATH_SHAPES)
def test_score_spikes(sattn, dev, shape):
    T, hq, hkv = shape
    note(f"score spikes T={T} Hq={hq} Hkv={hkv}")
    x, (k1, k2) = spiked(T, hq, hkv, seed=22)
    around = [k + d for k in (k1, k2) for d in (-1, 0, 1, 2, 31, 32, 63, 64)]
    around += [(k2 // 64) * 64 + d for d in (0, 31, 32, 63)]
    O, L = compare(sattn, dev, x, f"spikes T={T}", extra_rows=around)
    # past the second spike the weights are all on it: O is that V row
    G = hq // hkv
    for h in range(hq):
        v2 = x.Vt[h // G, :, k2].astype(np.float64)
        assert np.abs(O[k2:, h * 64:(h + 1) * 64] - v2[None, :]).max() <= TOL_O


@pytest.mark.parametrize("shape", [(4095, 32, 8), (8192, 16, 8), (8192, 16, 16),
                                   (4000, 32, 8), (3969, 32, 8)])
def test_eight_wave_shapes(sattn, dev, shape):
    """T=4000 and 3969 give 125 query blocks: the middle block has no light
    partner and the last slot group's second slot is empty (3969 also takes
    the scalar V^T staging)."""
    T, hq, hkv = shape
    note(f"eight-wave grid T={T} Hq={hq} Hkv={hkv}")
    x = make_inputs(T, hq, hkv, seed=23, peaked_fraction=0.01)
    compare(sattn, dev, x, f"T={T} Hq={hq} Hkv={hkv}")


@pytest.mark.parametrize("shape", [(8191, 2, 1), (8192, 4, 2)])
def test_split_key_long_sequences(sattn, dev, shape):
    """Grids too small for the main kernel at long T: each wave of the
    split-key kernel walks up to 32 key tiles through its own LDS region and
    the four partials are merged; T % 8 != 0 takes the scalar V^T staging."""
    T, hq, hkv = shape
    note(f"split-key kernel, long sequence T={T} Hq={hq} Hkv={hkv}")
    x = make_inputs(T, hq, hkv, seed=24, qk_std=1.25)
    compare(sattn, dev, x, f"split-key T={T} Hq={hq} Hkv={hkv}")


@pytest.mark.parametrize("shape", [(2048, 4, 4), (8008, 1, 1), (1000, 8, 8)])
def test_split_key_lds_staged(sattn, dev, shape):
    """Grids of at most one workgroup per CU with whole 16-byte V chunks take
    the split-key kernel's direct-to-LDS staging (two buffers a wave, the
    loads' waits counted by hand): waves walk up to 32 tiles, alternating the
    buffers, with ragged last tiles (T=8008, 1000).  Whole outputs against the
    oracle, and the V-rows entry bit-identical on the same values."""
    import torch
    T, hq, hkv = shape
    note(f"split-key kernel, LDS-staged T={T} Hq={hq} Hkv={hkv}")
    x = make_inputs(T, hq, hkv, seed=25, peaked_fraction=0.01)
    O, L = run(sattn, dev, x)
    Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
    assert_close(O, L, Or, Lr, f"LDS-staged split-key T={T} Hq={hq} Hkv={hkv}")
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    v = torch.from_numpy(np.ascontiguousarray(x.Vt.transpose(0, 2, 1))).to(dev)
    O2, L2 = sattn.fwd_vrows(q, k, v, x.c)
    torch.cuda.synchronize()
    assert np.array_equal(O2.cpu().numpy().astype(np.float64), O)
    assert np.array_equal(L2.cpu().numpy().astype(np.float64), L)


@pytest.mark.parametrize("shape", [(1024, 8, 2), (1000, 16, 4)])
def test_split_key_gqa_replication_bitwise(sattn, dev, shape):
    """The split-key kernels (LDS-staged at T=1024 Hq=8, register-staged at
    T=1000 Hq=16): K and V^T repeated per query head give bit-identical O and
    L."""
    import torch
    T, hq, hkv = shape
    note(f"split-key GQA replication T={T} Hq={hq} Hkv={hkv} vs Hkv={hq}")
    x = make_inputs(T, hq, hkv, seed=42)
    q, k, vt = (torch.from_numpy(a).to(dev) for a in (x.Q, x.K, x.Vt))
    O1, L1 = sattn.fwd(q, k, vt, x.c)
    G = hq // hkv
    O2, L2 = sattn.fwd(q, k.repeat_interleave(G, 0).contiguous(),
                       vt.repeat_interleave(G, 0).contiguous(), x.c)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
