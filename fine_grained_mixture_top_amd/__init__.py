"""Fine-grained MoE layer (routing, gather-fused grouped GEMMs, aggregation,
memory-efficient backward) in hand-written HIP for MI355X (gfx950).

The compute path lives in the shared library built from ``csrc/`` and is
reached through the C ABI declared in ``include/moe.h``; ``binding`` is a thin
ctypes layer over it.  ``inputs`` draws the seeded synthetic workloads.
"""
__all__ = ["inputs", "binding"]
