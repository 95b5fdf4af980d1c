"""The materialised path's C-ABI validation on the CPU (fake, never
dereferenced addresses; no device call)."""
import math

import pytest

from test_abi import sattn  # noqa: F401  (module fixture: builds and loads the library)

T, HQ, HKV = 256, 8, 2
GAP = 1 << 32
A = {name: (1 << 42) + i * GAP for i, name in enumerate(["Q", "K", "Vt", "O", "L", "S", "P"])}
C = 0.18033688


def full(sattn, t=T, hq=HQ, hkv=HKV, c=C, **kw):
    a = {**A, **kw}
    return sattn.sattn_mat_fwd_check(a["Q"], a["K"], a["Vt"], a["O"], a["L"], a["S"], a["P"], c,
                                     t, hq, hkv)


def test_valid(sattn):
    assert full(sattn) == sattn.SATTN_OK
    assert full(sattn, t=1) == sattn.SATTN_OK
    assert full(sattn, t=1000, hq=16, hkv=4) == sattn.SATTN_OK


@pytest.mark.parametrize("field", ["Q", "K", "Vt", "O", "L", "S", "P"])
def test_null(sattn, field):
    assert full(sattn, **{field: None}) == sattn.SATTN_ERR_NULL


@pytest.mark.parametrize("kw", [dict(t=0), dict(hq=6, hkv=4), dict(t=1 << 20, hq=1, hkv=1)])
def test_shape(sattn, kw):
    # the planes may not exceed 2^40 bytes (T = 2^20: 4 TiB)
    assert full(sattn, **kw) == sattn.SATTN_ERR_SHAPE


@pytest.mark.parametrize("c", [0.0, -1.0, math.inf, math.nan])
def test_scale(sattn, c):
    assert full(sattn, c=c) == sattn.SATTN_ERR_SCALE


@pytest.mark.parametrize("kw", [dict(S=A["S"] + 8), dict(P=A["P"] + 4), dict(O=A["O"] + 2),
                                dict(L=A["L"] + 2)])
def test_alignment(sattn, kw):
    assert full(sattn, **kw) == sattn.SATTN_ERR_ALIGN


@pytest.mark.parametrize("kw", [dict(S=A["Q"]), dict(P=A["S"] + 16), dict(O=A["P"] + 32),
                                dict(L=A["K"] + 16)])
def test_alias(sattn, kw):
    assert full(sattn, **kw) == sattn.SATTN_ERR_ALIAS


def test_step_checks_and_entries_validate_first(sattn):
    a = A
    assert sattn.sattn_mat_scores_check(a["Q"], a["K"], a["S"], C, T, HQ, HKV) == sattn.SATTN_OK
    assert sattn.sattn_mat_scores_check(a["Q"], a["K"], a["Q"], C, T, HQ, HKV) == sattn.SATTN_ERR_ALIAS
    assert sattn.sattn_mat_softmax_check(a["S"], a["P"], a["L"], T, HQ) == sattn.SATTN_OK
    assert sattn.sattn_mat_softmax_check(a["S"], a["S"], a["L"], T, HQ) == sattn.SATTN_ERR_ALIAS
    assert sattn.sattn_mat_pv_check(a["P"], a["Vt"], a["O"], T, HQ, HKV) == sattn.SATTN_OK
    assert sattn.sattn_mat_pv_check(a["P"], a["Vt"], None, T, HQ, HKV) == sattn.SATTN_ERR_NULL
    assert sattn.sattn_mat_fwd(None, a["K"], a["Vt"], a["O"], a["L"], a["S"], a["P"], C, T, HQ,
                               HKV, None) == sattn.SATTN_ERR_NULL
    assert sattn.sattn_mat_scores(a["Q"], a["K"], a["S"], -C, T, HQ, HKV,
                                  None) == sattn.SATTN_ERR_SCALE
    assert sattn.sattn_mat_softmax(a["S"], a["P"], a["L"] + 2, T, HQ, None) == sattn.SATTN_ERR_ALIGN
    assert sattn.sattn_mat_pv(a["P"], a["Vt"], a["O"], 0, HQ, HKV, None) == sattn.SATTN_ERR_SHAPE
