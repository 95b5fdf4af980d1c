"""The forward with V given as rows ([Hkv][T][64], sattn_fwd_vrows) through the
C ABI: bit-identical to sattn_fwd on the same values (the V^T operand of P V
is the same binary16 data, read with the LDS transpose read instead of from a
V^T tile) and within the forward's tolerance of the float64 oracle, across the
workgroup shapes (four- and eight-wave), GQA groups and ragged T."""
import numpy as np
import pytest

from causal_attention_forward_amd.inputs import make_inputs, make_workload
from oracle import attention_ref, attention_rows_ref
from parity_util import TOL_L, TOL_O, assert_close, note, sample_rows

pytestmark = pytest.mark.gpu


def both(sattn, dev, x):
    import torch
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    v = torch.from_numpy(np.ascontiguousarray(x.Vt.transpose(0, 2, 1))).to(dev)
    O1, L1 = sattn.fwd(q, k, vt, x.c)
    O2, L2 = sattn.fwd_vrows(q, k, v, x.c)
    torch.cuda.synchronize()
    return (O1.cpu().numpy(), L1.cpu().numpy(), O2.cpu().numpy(), L2.cpu().numpy())


SHAPES = [(1, 1, 1), (7, 2, 1), (64, 4, 2), (100, 3, 3), (257, 6, 2), (1000, 16, 4),
          (1023, 8, 8), (4095, 32, 8), (8192, 16, 16), (8192, 4, 2)]


@pytest.mark.parametrize("T,Hq,Hkv", SHAPES, ids=[f"T{t}_Hq{a}_Hkv{b}" for t, a, b in SHAPES])
def test_vrows_matches_vt_path_and_oracle(sattn, dev, T, Hq, Hkv):
    note(f"vrows T={T} Hq={Hq} Hkv={Hkv}")
    x = make_inputs(T, Hq, Hkv, seed=70 + T % 13, peaked_fraction=0.01)
    O1, L1, O2, L2 = both(sattn, dev, x)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2), "V rows differ from the V^T path"
    if T * Hq <= 20000:
        Or, Lr = attention_ref(x.Q, x.K, x.Vt, x.c)
        assert_close(O2.astype(np.float64), L2.astype(np.float64), Or, Lr, f"T={T}")
    else:
        rng = np.random.default_rng(T)
        for h in (0, Hq - 1):
            rows = sample_rows(T, rng, extra=8)
            Or, Lr = attention_rows_ref(x.Q, x.K, x.Vt, x.c, h, rows)
            got = O2[rows, h * 64:(h + 1) * 64].astype(np.float64)
            assert np.abs(got - Or).max() <= TOL_O and np.abs(L2[h, rows] - Lr).max() <= TOL_L


def test_vrows_headline_workload_bit_identical(sattn, dev):
    x = make_workload(3)
    O1, L1, O2, L2 = both(sattn, dev, x)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
