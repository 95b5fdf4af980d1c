"""Shared pieces of the GPU parity tests: running the HIP path through the
binding, the element-wise tolerance check, and the rows sampled at sizes
where the full oracle would take too long.

Tolerances (stated for the attention forward): max |O - O_ref| <= 4e-3 and
max |L - L_ref| <= 2e-4 (base-2 units), element by element.
"""
import sys

import numpy as np

TOL_O = 4e-3
TOL_L = 2e-4


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(sattn, dev, x):
    import torch
    q = torch.from_numpy(x.Q).to(dev)
    k = torch.from_numpy(x.K).to(dev)
    vt = torch.from_numpy(x.Vt).to(dev)
    O, L = sattn.fwd(q, k, vt, x.c)
    torch.cuda.synchronize()
    return O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64)


def assert_close(O, L, Or, Lr, what):
    assert np.isfinite(O).all() and np.isfinite(L).all(), what
    eo = float(np.abs(O - Or).max())
    el = float(np.abs(L - Lr).max())
    note(f"  {what}: max|dO|={eo:.3e} max|dL|={el:.3e}")
    assert eo <= TOL_O, f"{what}: max|dO| = {eo}"
    assert el <= TOL_L, f"{what}: max|dL| = {el}"


def sample_rows(T, rng, extra=24):
    fixed = {0, 1, 2, 31, 32, 63, 64, 65, 127, 128, T // 2, T - 65, T - 64, T - 33, T - 2, T - 1}
    rows = sorted(r for r in fixed | set(rng.integers(0, T, extra).tolist()) if 0 <= r < T)
    return rows
