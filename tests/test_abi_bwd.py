"""The backward's C-ABI validation on the CPU: every invalid argument is
rejected before any device call (fake, never-dereferenced addresses)."""
import math

import pytest

from test_abi import sattn  # noqa: F401  (module fixture: builds and loads the library)

T, HQ, HKV = 256, 8, 2
HALF = T * 64 * 2          # one binary16 [T][64] head
WORD = T * 64 * 4          # one binary32 [T][64] head
GAP = 1 << 30
BASE = 1 << 42
A = {name: BASE + i * GAP for i, name in enumerate(
    ["Q", "K", "Vt", "O", "dO", "L", "dQ", "dK", "dVt", "D", "ws"])}
C, S = 0.18033688, 0.125


def need(t=T, hq=HQ, hkv=HKV):
    return 2 * hq * t * 64 * 4 if hq != hkv else 0


def full(sattn, t=T, hq=HQ, hkv=HKV, c=C, s=S, ws_bytes=None, **kw):
    a = {**A, **kw}
    wb = need(t, hq, hkv) if ws_bytes is None else ws_bytes
    return sattn.sattn_bwd_check(a["Q"], a["K"], a["Vt"], a["O"], a["dO"], a["L"], a["dQ"],
                                 a["dK"], a["dVt"], a["D"], a["ws"], wb, c, s, t, hq, hkv)


def test_workspace_size(sattn):
    assert sattn.sattn_bwd_workspace_bytes(T, HQ, HKV) == 2 * HQ * T * 64 * 4
    assert sattn.sattn_bwd_workspace_bytes(T, 4, 4) == 0
    assert sattn.sattn_bwd_workspace_bytes(0, 4, 2) == 0
    assert sattn.sattn_bwd_workspace_bytes(T, 6, 4) == 0


def test_valid(sattn):
    assert full(sattn) == sattn.SATTN_OK
    assert full(sattn, t=1000, hq=16, hkv=4) == sattn.SATTN_OK
    assert full(sattn, hq=4, hkv=4, ws=None, ws_bytes=0) == sattn.SATTN_OK   # no workspace for G=1
    assert full(sattn, K=A["Q"], Vt=A["Q"]) == sattn.SATTN_OK                # inputs may overlap


@pytest.mark.parametrize("field", ["Q", "K", "Vt", "O", "dO", "L", "dQ", "dK", "dVt", "D"])
def test_null(sattn, field):
    assert full(sattn, **{field: None}) == sattn.SATTN_ERR_NULL


def test_workspace_errors(sattn):
    assert full(sattn, ws=None) == sattn.SATTN_ERR_WORKSPACE
    assert full(sattn, ws_bytes=need() - 1) == sattn.SATTN_ERR_WORKSPACE


@pytest.mark.parametrize("kw", [dict(t=0), dict(hq=6, hkv=4), dict(hq=65536, hkv=1)])
def test_shape(sattn, kw):
    assert full(sattn, **kw) == sattn.SATTN_ERR_SHAPE


@pytest.mark.parametrize("kw", [dict(c=0.0), dict(c=math.nan), dict(s=0.0), dict(s=-1.0),
                                dict(s=math.inf), dict(s=math.nan)])
def test_scale(sattn, kw):
    assert full(sattn, **kw) == sattn.SATTN_ERR_SCALE


@pytest.mark.parametrize("kw", [dict(Q=A["Q"] + 8), dict(dO=A["dO"] + 2), dict(O=A["O"] + 4),
                                dict(L=A["L"] + 2), dict(dQ=A["dQ"] + 4), dict(dK=A["dK"] + 8),
                                dict(dVt=A["dVt"] + 4), dict(D=A["D"] + 2), dict(ws=A["ws"] + 8)])
def test_alignment(sattn, kw):
    assert full(sattn, **kw) == sattn.SATTN_ERR_ALIGN


@pytest.mark.parametrize("kw", [dict(dQ=A["Q"]), dict(dK=A["dQ"] + HQ * WORD - 16),
                                dict(dVt=A["L"]), dict(D=A["dO"] + 64), dict(ws=A["dK"]),
                                dict(dQ=A["ws"] + need() - 16), dict(D=A["dQ"] + 16)])
def test_alias(sattn, kw):
    assert full(sattn, **kw) == sattn.SATTN_ERR_ALIAS


def test_split_checks(sattn):
    a = A
    assert sattn.sattn_bwd_query_check(a["Q"], a["K"], a["Vt"], a["O"], a["dO"], a["L"], a["dQ"],
                                       a["D"], C, S, T, HQ, HKV) == sattn.SATTN_OK
    assert sattn.sattn_bwd_query_check(a["Q"], a["K"], a["Vt"], None, a["dO"], a["L"], a["dQ"],
                                       a["D"], C, S, T, HQ, HKV) == sattn.SATTN_ERR_NULL
    assert sattn.sattn_bwd_key_check(a["Q"], a["K"], a["Vt"], a["dO"], a["L"], a["D"], a["dK"],
                                     a["dVt"], a["ws"], need(), C, S, T, HQ, HKV) == sattn.SATTN_OK
    # the key launch reads D: it may not overlap its outputs
    assert sattn.sattn_bwd_key_check(a["Q"], a["K"], a["Vt"], a["dO"], a["L"], a["dK"], a["dK"],
                                     a["dVt"], a["ws"], need(), C, S, T, HQ,
                                     HKV) == sattn.SATTN_ERR_ALIAS
    assert sattn.sattn_bwd_key_check(a["Q"], a["K"], a["Vt"], a["dO"], a["L"], None, a["dK"],
                                     a["dVt"], a["ws"], need(), C, S, T, HQ,
                                     HKV) == sattn.SATTN_ERR_NULL


def test_entry_points_validate_before_any_device_call(sattn):
    a = A
    assert sattn.sattn_bwd(None, a["K"], a["Vt"], a["O"], a["dO"], a["L"], a["dQ"], a["dK"],
                           a["dVt"], a["D"], a["ws"], need(), C, S, T, HQ,
                           HKV) == sattn.SATTN_ERR_NULL
    assert sattn.sattn_bwd_query(a["Q"], a["K"], a["Vt"], a["O"], a["dO"], a["L"], a["dQ"],
                                 a["D"], C, -S, T, HQ, HKV) == sattn.SATTN_ERR_SCALE
    assert sattn.sattn_bwd_key(a["Q"], a["K"], a["Vt"], a["dO"], a["L"], a["D"], a["dK"],
                               a["dVt"], a["ws"], 16, C, S, T, HQ,
                               HKV) == sattn.SATTN_ERR_WORKSPACE


def noalloc(sattn, t=T, hq=HQ, hkv=HKV, c=C, s=S, **kw):
    a = {**A, **kw}
    return sattn.sattn_bwd_key_noalloc(a["Q"], a["K"], a["Vt"], a["dO"], a["L"], a["D"], a["dK"],
                                       a["dVt"], c, s, t, hq, hkv)


def test_noalloc_key_launch_validates_before_any_device_call(sattn):
    """sattn_bwd_key_noalloc rejects bad arguments as sattn_bwd_key does, and a
    problem whose workspace exceeds its static region with SATTN_ERR_SCRATCH,
    all before any HIP call (the addresses here are fake)."""
    assert noalloc(sattn, D=None) == sattn.SATTN_ERR_NULL
    assert noalloc(sattn, t=0) == sattn.SATTN_ERR_SHAPE
    assert noalloc(sattn, c=math.nan) == sattn.SATTN_ERR_SCALE
    assert noalloc(sattn, dK=A["dK"] + 4) == sattn.SATTN_ERR_ALIGN
    assert noalloc(sattn, dVt=A["dK"]) == sattn.SATTN_ERR_ALIAS
    limit = sattn.BWD_NOALLOC_MAX_BYTES
    # T=4096 Hq=32 Hkv=8 needs exactly the region; one more token does not fit
    assert need(4096, 32, 8) == limit
    assert noalloc(sattn, t=4097, hq=32, hkv=8) == sattn.SATTN_ERR_SCRATCH
    assert noalloc(sattn, t=1 << 20, hq=4, hkv=1) == sattn.SATTN_ERR_SCRATCH
