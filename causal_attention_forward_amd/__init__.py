"""Causal streaming-attention forward for AMD MI355X (gfx950).

The compute lives in the HIP library ``libsattn.so`` built from ``csrc/``;
``sattn`` is its thin ctypes binding.  Importing this package loads nothing:
``from causal_attention_forward_amd import sattn`` loads the library and fails
loudly if it is missing.
"""
