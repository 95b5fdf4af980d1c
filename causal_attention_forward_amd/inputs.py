"""Seeded synthetic inputs for the causal streaming-attention forward.

This module only draws numbers and lays them out; it holds none of the
method's arithmetic.  Both the HIP path (through its tests and the benchmark)
and the float64 oracle consume what it returns.

Layouts follow the StreamingAttentionSM86 page (header comment of the forward
realization): Q and K are binary16 ``[head][T][64]`` and V^T is binary16
``[head][64][T]``.  The scale constant c is the binary32 value nearest
(1/sqrt(64)) / ln 2, which is what the Graph page's ``cgStreamingScale``
builds from the binary32 log2(e) by lowering its exponent by three.

Recipe (the pages give none; this is the reading recorded in the design
notes):  ``numpy.random.default_rng(seed)``; Q, K and V drawn as float32
standard normals in that order with shapes ``[Hq][T][64]``, ``[Hkv][T][64]``
and ``[Hkv][T][64]``; each multiplied by its standard deviation; for the
peaked-row workload ceil(0.01*T) distinct key rows per K/V head (drawn after
V, without replacement) get +3.0 on all 64 elements; everything is rounded to
binary16 (round to nearest even) and V is transposed per head into V^T.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

HEAD_DIM = 64

# binary32 nearest 0.125 / ln 2 (= 0x3E38AA3B); an input, not a derived value.
SCALE_C = np.float32(0.125 / math.log(2.0))


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    Hq: int
    Hkv: int
    qk_std: float = 1.0
    v_std: float = 1.0
    peaked_fraction: float = 0.0  # fraction of key rows given +peak_offset
    peak_offset: float = 3.0


# The five synthetic workloads the measurements are quoted on.
WORKLOADS = (
    Workload("tiny T=128 Hq=1 Hkv=1", 128, 1, 1),
    Workload("T=1024 Hq=8 Hkv=8 sd0.5", 1024, 8, 8, qk_std=0.5, v_std=0.5),
    Workload("ragged T=1000 Hq=16 Hkv=4 peaked", 1000, 16, 4, peaked_fraction=0.01),
    Workload("T=4096 Hq=32 Hkv=8", 4096, 32, 8),
    Workload("long T=16384 Hq=8 Hkv=2 qk-sd1.5", 16384, 8, 2, qk_std=1.5),
)


@dataclass
class Inputs:
    Q: np.ndarray   # float16 [Hq][T][64]
    K: np.ndarray   # float16 [Hkv][T][64]
    Vt: np.ndarray  # float16 [Hkv][64][T]
    c: np.float32
    T: int
    Hq: int
    Hkv: int


def make_inputs(T: int, Hq: int, Hkv: int, seed: int, *, qk_std: float = 1.0,
                v_std: float = 1.0, peaked_fraction: float = 0.0,
                peak_offset: float = 3.0, c: np.float32 = SCALE_C) -> Inputs:
    """Draw one seeded input set following the recipe in the module docstring."""
    if T < 0 or Hq < 1 or Hkv < 1:
        raise ValueError("need T >= 0, Hq >= 1, Hkv >= 1")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, T, HEAD_DIM), dtype=np.float32) * np.float32(qk_std)
    k = rng.standard_normal((Hkv, T, HEAD_DIM), dtype=np.float32) * np.float32(qk_std)
    v = rng.standard_normal((Hkv, T, HEAD_DIM), dtype=np.float32) * np.float32(v_std)
    if peaked_fraction > 0.0 and T > 0:
        n = int(math.ceil(peaked_fraction * T))
        for kv in range(Hkv):
            rows = rng.choice(T, size=n, replace=False)
            k[kv, rows, :] += np.float32(peak_offset)
    Q = q.astype(np.float16)
    K = k.astype(np.float16)
    Vt = np.ascontiguousarray(v.astype(np.float16).transpose(0, 2, 1))
    return Inputs(Q=np.ascontiguousarray(Q), K=np.ascontiguousarray(K), Vt=Vt,
                  c=np.float32(c), T=T, Hq=Hq, Hkv=Hkv)


def make_workload(index: int, seed: int | None = None) -> Inputs:
    """Inputs of workload ``index`` (0..4); the seed defaults to the index."""
    w = WORKLOADS[index]
    return make_inputs(w.T, w.Hq, w.Hkv, index if seed is None else seed,
                       qk_std=w.qk_std, v_std=w.v_std,
                       peaked_fraction=w.peaked_fraction, peak_offset=w.peak_offset)


def make_output_gradient(T: int, Hq: int, seed: int, *, std: float = 1.0) -> np.ndarray:
    """The output gradient dO for the backward: binary16, token-major
    ``[T][Hq*64]`` like the forward's O (element (i, h, d) at i*Hq*64 + h*64 + d).

    Recipe: ``numpy.random.default_rng([seed, 68])`` (a stream separate from
    the one ``make_inputs`` draws Q, K, V from for the same seed); float32
    standard normals of shape ``[T][Hq*64]`` times ``std``, rounded to binary16.
    """
    if T < 0 or Hq < 1:
        raise ValueError("need T >= 0, Hq >= 1")
    rng = np.random.default_rng([seed, 68])
    g = rng.standard_normal((T, Hq * HEAD_DIM), dtype=np.float32) * np.float32(std)
    return np.ascontiguousarray(g.astype(np.float16))
