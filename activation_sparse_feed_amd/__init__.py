"""Activation-sparse gated FFN forward for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libsffn.so`` built from ``csrc/``; the
Python layer in ``sffn`` only marshals torch device buffers and the current
stream into its C entry points.  ``workloads`` draws seeded synthetic inputs.
"""
__all__ = ["sffn", "workloads"]
