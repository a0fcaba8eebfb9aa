"""MI355X-native DFlash block-diffusion drafter round.

The compute path is the HIP library ``libdflash.so`` built from ``csrc/`` (entry
points declared in ``include/dflash.h``); ``binding`` is its thin ctypes
binding. ``config`` and ``synth`` hold shapes and seeded synthetic inputs only.
"""
from . import config  # noqa: F401

__all__ = ["config"]
