"""RotateAttention INT4 FlashAttention forward for AMD MI355X (gfx950).

The compute path lives in ``csrc/`` (HIP kernels behind a C ABI, built into
``librotattn.so``); ``rotattn`` is the thin ctypes binding over it and
``synth`` draws the seeded synthetic inputs.  Importing this package loads
nothing: ``from video_diffusion_transformers_amd import rotattn`` loads the
shared library and fails loudly if it has not been built.
"""

__all__ = ["rotattn", "synth"]
