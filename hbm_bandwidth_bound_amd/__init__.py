"""Batch-1 decode engine for one MI355X (gfx950): a persistent decode monokernel behind a C ABI.

Submodules are imported on demand so that the input generator (``synth``) can be used without
loading the GPU library.
"""
__version__ = "0.1.0"
