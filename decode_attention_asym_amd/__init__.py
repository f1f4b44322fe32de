"""decode_attention_asym_amd -- KIVI-style asymmetric low-bit KV cache and
in-loop-dequant decode attention for AMD MI355X (gfx950).

The compute path lives in ``libkvq.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/kvq.h``); ``kvq`` is its thin ctypes binding.
``configs`` and ``synth`` describe and generate the synthetic workloads.
"""
from . import configs, synth  # noqa: F401

__all__ = ["configs", "synth"]
