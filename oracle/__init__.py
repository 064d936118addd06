"""Reference oracle for the block-diffusion draft + verify step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (the HIP library and its Python binding) never imports,
calls or links it, and shares no code with it.
"""
from .dflash_oracle import *  # noqa: F401,F403
