"""MI355X (gfx950) hybrid gated-linear + sliding-window attention.

The compute path is the HIP library ``libglahybrid.so`` (C ABI in
``include/glahybrid.h``); ``binding`` marshals torch tensors into its entry
points.  Importing this package loads nothing: ``binding`` loads the library on
first use and raises if it has not been built.
"""
__all__ = ["binding", "inputs"]
