"""The C-ABI boundary on the CPU: the library loads, exports every function
include/sattn.h declares, and rejects every invalid argument before touching a
device (no kernel is launched by any test here)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sattn.h")
LIB = os.path.join(ROOT, "causal_attention_forward_amd", "libsattn.so")


@pytest.fixture(scope="module")
def sattn():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    from causal_attention_forward_amd import sattn as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[\w ]*?[\w*]\s*\*?\s*(sattn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted([
        "sattn_fwd", "sattn_fwd_vrows", "sattn_fwd_check", "sattn_status_string", "sattn_bwd",
        "sattn_bwd_check",
        "sattn_bwd_key", "sattn_bwd_key_check", "sattn_bwd_key_noalloc", "sattn_bwd_query",
        "sattn_bwd_query_check",
        "sattn_bwd_workspace_bytes", "sattn_mat_fwd", "sattn_mat_fwd_check",
        "sattn_mat_scores", "sattn_mat_softmax", "sattn_mat_pv", "sattn_mat_scores_check",
        "sattn_mat_softmax_check", "sattn_mat_pv_check"])


def test_library_exports_every_declared_symbol(sattn):
    lib = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(sattn.EXPORTS) == set(declared_functions())


def test_status_strings(sattn):
    for s in range(10):
        text = sattn.sattn_status_string(s)
        assert text and text != "unknown sattn status"
    assert sattn.sattn_status_string(10) == "unknown sattn status"
    assert sattn.sattn_status_string(-1) == "unknown sattn status"


# Fake, never-dereferenced addresses laid out without overlap.
T, HQ, HKV = 256, 8, 2
PLANE = T * 64 * 2
BASE = 1 << 40
Qa = BASE
Ka = Qa + HQ * PLANE
Va = Ka + HKV * PLANE
Oa = Va + HKV * PLANE
La = Oa + HQ * PLANE
C = 0.18033688


def check(sattn, Q=Qa, K=Ka, V=Va, O=Oa, L=La, c=C, t=T, hq=HQ, hkv=HKV):
    return sattn.sattn_fwd_check(Q, K, V, O, L, c, t, hq, hkv)


def test_valid_arguments_pass(sattn):
    assert check(sattn) == sattn.SATTN_OK
    assert check(sattn, t=1) == sattn.SATTN_OK
    far = 1 << 44
    spaced = dict(Q=far, K=far + (1 << 36), V=far + (2 << 36), O=far + (3 << 36), L=far + (4 << 36))
    assert check(sattn, t=1000, hq=16, hkv=4, **spaced) == sattn.SATTN_OK  # ragged T is admitted


@pytest.mark.parametrize("field", ["Q", "K", "V", "O", "L"])
def test_null_pointers(sattn, field):
    assert check(sattn, **{field: None}) == sattn.SATTN_ERR_NULL


@pytest.mark.parametrize("kw", [dict(t=0), dict(t=-5), dict(hq=0), dict(hkv=0), dict(hq=-1),
                                dict(hq=8, hkv=3), dict(hq=6, hkv=4), dict(hq=65536, hkv=1),
                                dict(hq=64, t=1 << 18)])
def test_bad_shapes(sattn, kw):
    assert check(sattn, **kw) == sattn.SATTN_ERR_SHAPE


def test_size_limit_is_the_pages_bound(sattn):
    # Hq*64*T*4 <= 2^32-1: T = 2^24/Hq... with Hq=1: T = 2^24 - 1 admitted, 2^24 refused
    far = 1 << 44
    ok = sattn.sattn_fwd_check(far, far + (1 << 36), far + (2 << 36), far + (3 << 36),
                               far + (4 << 36), C, (1 << 24) - 1, 1, 1)
    assert ok == sattn.SATTN_OK
    bad = sattn.sattn_fwd_check(far, far + (1 << 36), far + (2 << 36), far + (3 << 36),
                                far + (4 << 36), C, 1 << 24, 1, 1)
    assert bad == sattn.SATTN_ERR_SHAPE


@pytest.mark.parametrize("c", [0.0, -0.18, math.inf, -math.inf, math.nan])
def test_bad_scale(sattn, c):
    assert check(sattn, c=c) == sattn.SATTN_ERR_SCALE


@pytest.mark.parametrize("kw", [dict(Q=Qa + 2), dict(K=Ka + 8), dict(V=Va + 4), dict(O=Oa + 2),
                                dict(L=La + 2)])
def test_misalignment(sattn, kw):
    assert check(sattn, **kw) == sattn.SATTN_ERR_ALIGN


def test_four_byte_aligned_L_is_fine(sattn):
    assert check(sattn, L=La + 4) == sattn.SATTN_OK


@pytest.mark.parametrize("kw", [dict(O=Qa), dict(O=Ka + 16), dict(O=Va - HQ * PLANE + 16),
                                dict(L=Oa + 64), dict(L=Qa), dict(L=Va + 1024),
                                dict(O=La - HQ * PLANE + 16)])
def test_aliasing(sattn, kw):
    assert check(sattn, **kw) == sattn.SATTN_ERR_ALIAS


def test_inputs_may_overlap_each_other(sattn):
    assert check(sattn, K=Qa, V=Qa) == sattn.SATTN_OK


def test_entry_point_validates_before_any_device_call(sattn):
    # Invalid arguments return their status without a HIP call, so this runs
    # on a machine with no GPU.
    assert sattn.sattn_fwd(None, Ka, Va, Oa, La, C, T, HQ, HKV, None) == sattn.SATTN_ERR_NULL
    assert sattn.sattn_fwd(Qa, Ka, Va, Oa, La, C, 0, HQ, HKV, None) == sattn.SATTN_ERR_SHAPE
    assert sattn.sattn_fwd(Qa, Ka, Va, Oa, La, -1.0, T, HQ, HKV, None) == sattn.SATTN_ERR_SCALE
    assert sattn.sattn_fwd(Qa, Ka, Va, Qa, La, C, T, HQ, HKV, None) == sattn.SATTN_ERR_ALIAS
    assert sattn.sattn_fwd_vrows(None, Ka, Va, Oa, La, C, T, HQ, HKV, None) == sattn.SATTN_ERR_NULL
    assert sattn.sattn_fwd_vrows(Qa, Ka, Va + 8, Oa, La, C, T, HQ, HKV, None) == sattn.SATTN_ERR_ALIGN
    assert sattn.sattn_fwd_vrows(Qa, Ka, Va, Va, La, C, T, HQ, HKV, None) == sattn.SATTN_ERR_ALIAS


def test_product_path_has_no_oracle_or_fallback():
    # the product package never imports the oracle, and the binding loads the
    # HIP library unconditionally
    pkg = os.path.join(ROOT, "causal_attention_forward_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(from|import)\s+oracle", src, flags=re.M), name
            assert "importlib" not in src, name
    src = open(os.path.join(pkg, "sattn.py")).read()
    assert "raise ImportError" in src


def test_binding_loads_a_single_hip_runtime():
    """Importing the binding before torch must not map a second HIP runtime
    next to torch's own (two runtimes driving one GPU crash the process)."""
    import subprocess
    import sys
    code = ("from causal_attention_forward_amd import sattn\n"
            "import torch\n"
            "print(len(sattn.hip_runtimes_loaded()))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1"
