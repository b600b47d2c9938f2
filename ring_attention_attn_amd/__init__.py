"""MI355X-native ring-step attention (one GPU's share of context-parallel causal
GQA attention): hand-written HIP kernels for gfx950 behind a C ABI
(``libringattn.so``), with a thin ctypes binding of the same names.

Import of this package does not load the native library; ``binding`` does, and
fails loudly if it has not been built.
"""
__all__ = ["binding", "ring", "synth", "configs"]
