"""RACE attention (soft-LSH sketch attention) for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``librace_attn.so`` (hand-written HIP
kernels, declared in ``include/race_attn.h``); ``sketch_attention_soft_amd.binding``
is a thin ctypes layer over it that takes torch device tensors.  Importing
this package does not load the library; the binding loads it on first use
and raises if it is missing.
"""

__all__ = ["binding", "inputs"]
