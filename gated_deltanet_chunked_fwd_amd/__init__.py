"""MI355X-native Gated DeltaNet chunked-prefill forward (gfx950 HIP kernels behind a C ABI).

The compute lives in ``libgdn.so`` (built from ``csrc/``); ``binding`` marshals
torch tensors into its C entry points.  ``synth`` holds the seeded input
generators.  Importing the package loads nothing; the first call into
``binding`` loads the library and raises if it is missing.
"""
__all__ = ["binding", "synth"]
