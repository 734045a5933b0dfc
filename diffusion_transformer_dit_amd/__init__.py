"""libdit_block: forward pass of a Flux-style single-stream DiT block on
MI355X (gfx950), hand-written HIP kernels behind a C ABI.

The compute path is the shared library ``libdit_block.so`` (built by
``python -m diffusion_transformer_dit_amd.build``); ``binding`` is its thin
ctypes wrapper.  Importing ``binding`` fails loudly when the library is
missing: there is no fallback path.
"""
__all__ = ["binding", "build"]
__version__ = "0.1.0"
