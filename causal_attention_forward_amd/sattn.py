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
_lib.sattn_fwd_check.restype = ctypes.c_int
_lib.sattn_fwd_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int]
_lib.sattn_status_string.restype = ctypes.c_char_p
_lib.sattn_status_string.argtypes = [ctypes.c_int]

SATTN_OK = 0
SATTN_ERR_NULL = 1
SATTN_ERR_SHAPE = 2
SATTN_ERR_SCALE = 3
SATTN_ERR_ALIGN = 4
SATTN_ERR_ALIAS = 5
SATTN_ERR_DEVICE = 6
SATTN_ERR_LAUNCH = 7
HEAD_DIM = 64

EXPORTS = ("sattn_fwd", "sattn_fwd_check", "sattn_status_string")


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


def sattn_fwd_check(Q: int, K: int, Vt: int, O: int, L: int, c: float, T: int, Hq: int,
                    Hkv: int) -> int:
    """Host-side validation only (no HIP call); returns the status code."""
    return _lib.sattn_fwd_check(Q, K, Vt, O, L, ctypes.c_float(c), T, Hq, Hkv)


def fwd(q, k, vt, c, out=None, lse=None, stream=None):
    """Attention forward on torch tensors already on the GPU.

    q: float16 [Hq][T][64], k: float16 [Hkv][T][64], vt: float16 [Hkv][64][T],
    all contiguous on one device.  Returns ``(O, L)``: float16 [T][Hq*64] and
    float32 [Hq][T] (allocated here unless ``out`` / ``lse`` are given).  The
    kernel is enqueued on ``stream`` (default: torch's current stream).
    """
    import torch

    Hq, T, D = q.shape
    Hkv = k.shape[0]
    if D != HEAD_DIM or tuple(k.shape) != (Hkv, T, D) or tuple(vt.shape) != (Hkv, D, T):
        raise ValueError(f"shapes q{tuple(q.shape)} k{tuple(k.shape)} vt{tuple(vt.shape)}")
    for name, x in (("q", q), ("k", k), ("vt", vt)):
        if x.dtype != torch.float16 or not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float16 GPU tensor")
    if out is None:
        out = torch.empty((T, Hq * D), dtype=torch.float16, device=q.device)
    if lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
    if (out.dtype != torch.float16 or lse.dtype != torch.float32 or not out.is_contiguous()
            or not lse.is_contiguous() or out.numel() != T * Hq * D or lse.numel() != Hq * T):
        raise ValueError("out must be contiguous float16 [T][Hq*64], lse contiguous float32 [Hq][T]")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        st = sattn_fwd(q.data_ptr(), k.data_ptr(), vt.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       float(c), T, Hq, Hkv, stream.cuda_stream)
    if st != SATTN_OK:
        raise SattnError(st)
    return out, lse
