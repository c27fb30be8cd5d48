"""librescomp: residual compression with error feedback for parallel diffusion
inference, as hand-written HIP kernels for gfx950 behind a small C ABI.

Submodules:
  librescomp -- ctypes binding of the C ABI (loads the HIP library; fails loudly
                when it is not built).
  synth      -- seeded synthetic activation sequences (inputs only).
  build      -- compiles the HIP library for gfx950.
"""
