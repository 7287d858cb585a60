"""Kamera relocate + patch operator for AMD Instinct MI355X (gfx950).

``KV(B|A) ~= R(delta) KV(B|empty) + U_m V_m^T`` in place over MHA/GQA/MLA KV caches,
contiguous or paged, through the C ABI of ``libkamera.so`` (include/kamera.h).

- ``kamera``: ctypes binding with the C entry-point names, plus descriptor helpers.
- ``synth``: seeded synthetic workloads, layouts and byte accounting.
- ``ops``: torch-tensor front end (fills descriptors; the kernels do the work).
"""
from . import synth  # noqa: F401

__all__ = ["kamera", "synth", "ops"]
