"""MI355X (gfx950) Groth16 H-polynomial pipeline over the BN254 scalar field.

The compute path is libg16.so (hand-written HIP, include/g16.h); `binding` is its
ctypes wrapper over torch device memory and streams, and `synth` draws the seeded
synthetic inputs.  Importing the package does not load the library; the first call
does, and raises if it has not been built.
"""
from . import binding, synth  # noqa: F401

__all__ = ["binding", "synth"]
