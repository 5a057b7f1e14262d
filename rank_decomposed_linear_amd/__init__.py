"""Decomposed-layer forward pass on MI355X (gfx950).

Submodules:
  workloads -- seeded synthetic workload shapes and inputs (numpy only)
  binding   -- ctypes binding of libdlayer.so, the HIP library (needs torch)
  build     -- hipcc build of libdlayer.so
"""
__all__ = ["workloads", "binding", "build"]
