"""MI355X (gfx950) block-diffusion draft + verify hot path.

Submodules:
  _binding  ctypes binding of libdflash.so (the C ABI of include/dflash.h)
  drafter   device-memory owner that calls the C ABI (PyTorch for memory/streams)
  synth     seeded synthetic shapes and inputs
  build     hipcc build of libdflash.so
Importing ``_binding`` or ``drafter`` requires the built library.
"""
