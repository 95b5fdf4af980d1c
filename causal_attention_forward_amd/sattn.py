"""ctypes binding of libsattn: argument marshalling only.

Every step of the attention runs in the HIP library; this module converts
torch device tensors to pointers and sizes, picks the current stream, and
turns status codes into exceptions.  Importing it loads ``libsattn.so`` from
this package directory and raises ``ImportError`` if it is missing: there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os

# torch owns the device memory and streams handed to the library, so its HIP
# runtime must be the one libsattn binds to.  torch ships its own
# libamdhip64; importing torch first makes the loader resolve libsattn's
# dependency to that already-loaded runtime instead of mapping a second one.
import torch  # noqa: E402,F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")

_lib = ctypes.CDLL(LIB_PATH)


def hip_runtimes_loaded():
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if len(hip_runtimes_loaded()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process "
                      f"({hip_runtimes_loaded()}); load libsattn only through this module")

# names and signatures as declared in include/sattn.h
_lib.sattn_fwd.restype = ctypes.c_int
_lib.sattn_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                           ctypes.c_int, ctypes.c_void_p]
_lib.sattn_fwd_vrows.restype = ctypes.c_int
_lib.sattn_fwd_vrows.argtypes = _lib.sattn_fwd.argtypes
_lib.sattn_fwd_check.restype = ctypes.c_int
_lib.sattn_fwd_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.sattn_status_string.restype = ctypes.c_char_p
_lib.sattn_status_string.argtypes = [ctypes.c_int]
_P, _F, _I, _U64 = ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_ulonglong
_lib.sattn_mat_fwd.restype = ctypes.c_int
_lib.sattn_mat_fwd.argtypes = [_P] * 7 + [_F, _I, _I, _I, _P]
_lib.sattn_mat_scores.restype = ctypes.c_int
_lib.sattn_mat_scores.argtypes = [_P] * 3 + [_F, _I, _I, _I, _P]
_lib.sattn_mat_softmax.restype = ctypes.c_int
_lib.sattn_mat_softmax.argtypes = [_P] * 3 + [_I, _I, _P]
_lib.sattn_mat_pv.restype = ctypes.c_int
_lib.sattn_mat_pv.argtypes = [_P] * 3 + [_I, _I, _I, _P]
_lib.sattn_mat_scores_check.restype = ctypes.c_int
_lib.sattn_mat_scores_check.argtypes = [_P] * 3 + [_F, _I, _I, _I]
_lib.sattn_mat_softmax_check.restype = ctypes.c_int
_lib.sattn_mat_softmax_check.argtypes = [_P] * 3 + [_I, _I]
_lib.sattn_mat_pv_check.restype = ctypes.c_int
_lib.sattn_mat_pv_check.argtypes = [_P] * 3 + [_I, _I, _I]
_lib.sattn_mat_fwd_check.restype = ctypes.c_int
_lib.sattn_mat_fwd_check.argtypes = [_P] * 7 + [_F, _I, _I, _I]
_lib.sattn_bwd_query.restype = ctypes.c_int
_lib.sattn_bwd_query.argtypes = [_P] * 8 + [_F, _F, _I, _I, _I, _P]
_lib.sattn_bwd_key.restype = ctypes.c_int
_lib.sattn_bwd_key.argtypes = [_P] * 9 + [_U64, _F, _F, _I, _I, _I, _P]
_lib.sattn_bwd_key_noalloc.restype = ctypes.c_int
_lib.sattn_bwd_key_noalloc.argtypes = [_P] * 8 + [_F, _F, _I, _I, _I, _P]
_lib.sattn_bwd.restype = ctypes.c_int
_lib.sattn_bwd.argtypes = [_P] * 11 + [_U64, _F, _F, _I, _I, _I, _P]
_lib.sattn_bwd_workspace_bytes.restype = ctypes.c_ulonglong
_lib.sattn_bwd_workspace_bytes.argtypes = [_I, _I, _I]
_lib.sattn_bwd_check.restype = ctypes.c_int
_lib.sattn_bwd_check.argtypes = [_P] * 11 + [_U64, _F, _F, _I, _I, _I]
_lib.sattn_bwd_query_check.restype = ctypes.c_int
_lib.sattn_bwd_query_check.argtypes = [_P] * 8 + [_F, _F, _I, _I, _I]
_lib.sattn_bwd_key_check.restype = ctypes.c_int
_lib.sattn_bwd_key_check.argtypes = [_P] * 9 + [_U64, _F, _F, _I, _I, _I]

SATTN_OK = 0
SATTN_ERR_NULL = 1
SATTN_ERR_SHAPE = 2
SATTN_ERR_SCALE = 3
SATTN_ERR_ALIGN = 4
SATTN_ERR_ALIAS = 5
SATTN_ERR_DEVICE = 6
SATTN_ERR_LAUNCH = 7
SATTN_ERR_WORKSPACE = 8
SATTN_ERR_SCRATCH = 9
BWD_NOALLOC_MAX_BYTES = 64 << 20   # SATTN_BWD_NOALLOC_MAX_BYTES
HEAD_DIM = 64

EXPORTS = ("sattn_fwd", "sattn_fwd_vrows", "sattn_fwd_check", "sattn_status_string", "sattn_bwd_query",
           "sattn_bwd_key", "sattn_bwd_key_noalloc", "sattn_bwd", "sattn_bwd_workspace_bytes",
           "sattn_bwd_check",
           "sattn_bwd_query_check", "sattn_bwd_key_check", "sattn_mat_fwd",
           "sattn_mat_fwd_check", "sattn_mat_scores", "sattn_mat_softmax", "sattn_mat_pv",
           "sattn_mat_scores_check", "sattn_mat_softmax_check", "sattn_mat_pv_check")


class SattnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"sattn status {status}: {sattn_status_string(status)}")


def sattn_status_string(status: int) -> str:
    return _lib.sattn_status_string(int(status)).decode()


def sattn_fwd(Q: int, K: int, Vt: int, O: int, L: int, c: float, T: int, Hq: int, Hkv: int,
              stream: int | None = None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return _lib.sattn_fwd(Q, K, Vt, O, L, ctypes.c_float(c), T, Hq, Hkv, stream)


def sattn_fwd_vrows(Q: int, K: int, V: int, O: int, L: int, c: float, T: int, Hq: int, Hkv: int,
                    stream: int | None = None) -> int:
    """The C entry point taking V as rows [Hkv][T][64]; returns the status code."""
    return _lib.sattn_fwd_vrows(Q, K, V, O, L, ctypes.c_float(c), T, Hq, Hkv, stream)


def sattn_fwd_check(Q: int, K: int, Vt: int, O: int, L: int, c: float, T: int, Hq: int,
                    Hkv: int) -> int:
    """Host-side validation only (no HIP call); returns the status code."""
    return _lib.sattn_fwd_check(Q, K, Vt, O, L, ctypes.c_float(c), T, Hq, Hkv)


def _check_tensor(name, x, dtype, shape, device):
    """x must be a contiguous `dtype` tensor of `shape` on the GPU `device`:
    the library reads and writes through the raw address, so anything else
    would make the kernels touch memory that is not the tensor's."""
    import torch
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if (tuple(x.shape) != tuple(shape) or x.dtype != dtype or not x.is_cuda
            or not x.is_contiguous() or (device is not None and x.device != device)):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"on {device if device is not None else 'the GPU'} (got "
                         f"{x.dtype} {tuple(x.shape)} on {x.device}, "
                         f"contiguous={x.is_contiguous()})")


def _fwd_operands(q, k, v, v_shape_of, out, lse):
    """Checks of the forward's operands; allocates O and L when not given."""
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a float16 GPU tensor [Hq][T][64]")
    Hq, T, D = q.shape
    if not isinstance(k, torch.Tensor) or k.dim() != 3:
        raise ValueError("k must be a float16 GPU tensor [Hkv][T][64]")
    Hkv = k.shape[0]
    dev = q.device
    _check_tensor("q", q, torch.float16, (Hq, T, HEAD_DIM), None)
    _check_tensor("k", k, torch.float16, (Hkv, T, HEAD_DIM), dev)
    _check_tensor("v", v, torch.float16, v_shape_of(Hkv, T), dev)
    if out is None:
        out = torch.empty((T, Hq * D), dtype=torch.float16, device=dev)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    _check_tensor("out", out, torch.float16, (T, Hq * HEAD_DIM), dev)
    _check_tensor("lse", lse, torch.float32, (Hq, T), dev)
    return Hq, T, Hkv, out, lse


def fwd_vrows(q, k, v, c, out=None, lse=None, stream=None):
    """As ``fwd`` with V given as rows: v float16 [Hkv][T][64] (no V^T needed)."""
    import torch

    Hq, T, Hkv, out, lse = _fwd_operands(q, k, v, lambda hkv, t: (hkv, t, HEAD_DIM), out, lse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = sattn_fwd_vrows(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), float(c), T, Hq, Hkv, stream.cuda_stream)
    if st != SATTN_OK:
        raise SattnError(st)
    return out, lse


def fwd(q, k, vt, c, out=None, lse=None, stream=None):
    """Attention forward on torch tensors already on the GPU.

    q: float16 [Hq][T][64], k: float16 [Hkv][T][64], vt: float16 [Hkv][64][T],
    all contiguous on one device.  Returns ``(O, L)``: float16 [T][Hq*64] and
    float32 [Hq][T] (allocated here unless ``out`` / ``lse`` are given).  The
    kernel is enqueued on ``stream`` (default: torch's current stream).
    """
    import torch

    Hq, T, Hkv, out, lse = _fwd_operands(q, k, vt, lambda hkv, t: (hkv, HEAD_DIM, t), out, lse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = sattn_fwd(q.data_ptr(), k.data_ptr(), vt.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       float(c), T, Hq, Hkv, stream.cuda_stream)
    if st != SATTN_OK:
        raise SattnError(st)
    return out, lse


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def sattn_bwd_workspace_bytes(T: int, Hq: int, Hkv: int) -> int:
    return int(_lib.sattn_bwd_workspace_bytes(T, Hq, Hkv))


def sattn_bwd_check(Q, K, Vt, O, dO, L, dQ, dK, dVt, D, ws, ws_bytes, c, s, T, Hq, Hkv) -> int:
    """Host-side validation only (no HIP call); returns the status code."""
    return _lib.sattn_bwd_check(Q, K, Vt, O, dO, L, dQ, dK, dVt, D, ws, ws_bytes,
                                ctypes.c_float(c), ctypes.c_float(s), T, Hq, Hkv)


def sattn_bwd_query_check(Q, K, Vt, O, dO, L, dQ, D, c, s, T, Hq, Hkv) -> int:
    return _lib.sattn_bwd_query_check(Q, K, Vt, O, dO, L, dQ, D, ctypes.c_float(c),
                                      ctypes.c_float(s), T, Hq, Hkv)


def sattn_bwd_key_check(Q, K, Vt, dO, L, D, dK, dVt, ws, ws_bytes, c, s, T, Hq, Hkv) -> int:
    return _lib.sattn_bwd_key_check(Q, K, Vt, dO, L, D, dK, dVt, ws, ws_bytes, ctypes.c_float(c),
                                    ctypes.c_float(s), T, Hq, Hkv)


def sattn_bwd(Q, K, Vt, O, dO, L, dQ, dK, dVt, D, ws, ws_bytes, c, s, T, Hq, Hkv,
              stream=None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return _lib.sattn_bwd(Q, K, Vt, O, dO, L, dQ, dK, dVt, D, ws, ws_bytes, ctypes.c_float(c),
                          ctypes.c_float(s), T, Hq, Hkv, stream)


def sattn_bwd_query(Q, K, Vt, O, dO, L, dQ, D, c, s, T, Hq, Hkv, stream=None) -> int:
    return _lib.sattn_bwd_query(Q, K, Vt, O, dO, L, dQ, D, ctypes.c_float(c), ctypes.c_float(s),
                                T, Hq, Hkv, stream)


def sattn_bwd_key(Q, K, Vt, dO, L, D, dK, dVt, ws, ws_bytes, c, s, T, Hq, Hkv,
                  stream=None) -> int:
    return _lib.sattn_bwd_key(Q, K, Vt, dO, L, D, dK, dVt, ws, ws_bytes, ctypes.c_float(c),
                              ctypes.c_float(s), T, Hq, Hkv, stream)


def sattn_bwd_key_noalloc(Q, K, Vt, dO, L, D, dK, dVt, c, s, T, Hq, Hkv, stream=None) -> int:
    """The key launch with the library's static workspace (allocates nothing)."""
    return _lib.sattn_bwd_key_noalloc(Q, K, Vt, dO, L, D, dK, dVt, ctypes.c_float(c),
                                      ctypes.c_float(s), T, Hq, Hkv, stream)


def _out(x, shape, dev):
    import torch
    if x is None:
        return torch.empty(shape, dtype=torch.float32, device=dev)
    _check_tensor("output", x, torch.float32, shape, dev)
    return x


def bwd(q, k, vt, o, do, lse, c, s, dq=None, dk=None, dvt=None, D=None, workspace=None,
        stream=None):
    """Attention backward on torch GPU tensors (query launch, then key launch
    and the grouped reduction).

    q [Hq][T][64], k [Hkv][T][64], vt [Hkv][64][T], o and do [T][Hq*64]
    (float16, contiguous), lse float32 [Hq][T] (the forward's L); c the
    base-2 and s the natural score scale.  Returns ``(dQ, dK, dVt, D)``:
    float32 [Hq][T][64], [Hkv][T][64], [Hkv][64][T] and [Hq][T].  The
    workspace (uint8, at least ``sattn_bwd_workspace_bytes`` bytes) is
    allocated here unless given.
    """
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or not isinstance(k, torch.Tensor) \
            or k.dim() != 3:
        raise ValueError("q [Hq][T][64] and k [Hkv][T][64] must be float16 GPU tensors")
    Hq, T, _ = q.shape
    Hkv = k.shape[0]
    dev = q.device
    f16, f32 = torch.float16, torch.float32
    _check_tensor("q", q, f16, (Hq, T, HEAD_DIM), None)
    _check_tensor("k", k, f16, (Hkv, T, HEAD_DIM), dev)
    _check_tensor("vt", vt, f16, (Hkv, HEAD_DIM, T), dev)
    _check_tensor("o", o, f16, (T, Hq * HEAD_DIM), dev)
    _check_tensor("do", do, f16, (T, Hq * HEAD_DIM), dev)
    _check_tensor("lse", lse, f32, (Hq, T), dev)
    dq = _out(dq, (Hq, T, HEAD_DIM), dev)
    dk = _out(dk, (Hkv, T, HEAD_DIM), dev)
    dvt = _out(dvt, (Hkv, HEAD_DIM, T), dev)
    D = _out(D, (Hq, T), dev)
    need = sattn_bwd_workspace_bytes(T, Hq, Hkv)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda \
                or workspace.device != dev or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = sattn_bwd(q.data_ptr(), k.data_ptr(), vt.data_ptr(), o.data_ptr(), do.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dvt.data_ptr(),
                       D.data_ptr(), ws_ptr, ws_bytes, float(c), float(s), T, Hq, Hkv,
                       stream.cuda_stream)
    if st != SATTN_OK:
        raise SattnError(st)
    return dq, dk, dvt, D


# --------------------------------------------------------------------------
# materialised path
# --------------------------------------------------------------------------
def sattn_mat_fwd(Q, K, Vt, O, L, S, P, c, T, Hq, Hkv, stream=None) -> int:
    """The C entry point with raw device addresses; returns the status code."""
    return _lib.sattn_mat_fwd(Q, K, Vt, O, L, S, P, ctypes.c_float(c), T, Hq, Hkv, stream)


def sattn_mat_scores(Q, K, S, c, T, Hq, Hkv, stream=None) -> int:
    return _lib.sattn_mat_scores(Q, K, S, ctypes.c_float(c), T, Hq, Hkv, stream)


def sattn_mat_softmax(S, P, L, T, Hq, stream=None) -> int:
    return _lib.sattn_mat_softmax(S, P, L, T, Hq, stream)


def sattn_mat_pv(P, Vt, O, T, Hq, Hkv, stream=None) -> int:
    return _lib.sattn_mat_pv(P, Vt, O, T, Hq, Hkv, stream)


def sattn_mat_scores_check(Q, K, S, c, T, Hq, Hkv) -> int:
    return _lib.sattn_mat_scores_check(Q, K, S, ctypes.c_float(c), T, Hq, Hkv)


def sattn_mat_softmax_check(S, P, L, T, Hq) -> int:
    return _lib.sattn_mat_softmax_check(S, P, L, T, Hq)


def sattn_mat_pv_check(P, Vt, O, T, Hq, Hkv) -> int:
    return _lib.sattn_mat_pv_check(P, Vt, O, T, Hq, Hkv)


def sattn_mat_fwd_check(Q, K, Vt, O, L, S, P, c, T, Hq, Hkv) -> int:
    return _lib.sattn_mat_fwd_check(Q, K, Vt, O, L, S, P, ctypes.c_float(c), T, Hq, Hkv)


def mat_fwd(q, k, vt, c, scores=None, probs=None, out=None, lse=None, stream=None):
    """The materialised path on torch GPU tensors (layouts as ``fwd``).

    Returns ``(O, L, S, P)``: float16 [T][Hq*64], float32 [Hq][T], and the
    planes float32 / float16 [Hq][T][T] (entries above the diagonal are left
    as allocated).  Caller-given planes and outputs must be contiguous, of
    those dtypes and shapes, on q's device.
    """
    import torch
    Hq, T, Hkv, out, lse = _fwd_operands(q, k, vt, lambda hkv, t: (hkv, HEAD_DIM, t), out, lse)
    dev = q.device
    if scores is None:
        scores = torch.empty((Hq, T, T), dtype=torch.float32, device=dev)
    if probs is None:
        probs = torch.empty((Hq, T, T), dtype=torch.float16, device=dev)
    _check_tensor("scores", scores, torch.float32, (Hq, T, T), dev)
    _check_tensor("probs", probs, torch.float16, (Hq, T, T), dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        st = sattn_mat_fwd(q.data_ptr(), k.data_ptr(), vt.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), scores.data_ptr(), probs.data_ptr(), float(c), T, Hq,
                           Hkv, stream.cuda_stream)
    if st != SATTN_OK:
        raise SattnError(st)
    return out, lse, scores, probs
