"""Medusa verify step for AMD Instinct MI355X (gfx950).

The work happens in ``libmedusa_amd.so`` (HIP kernels behind the C ABI in
``include/medusa.h``); ``api`` is a thin ctypes binding over it and ``synth``
makes seeded synthetic inputs.  Importing the package does not load the
library; the first call into ``api`` does, and fails loudly if it is missing.
"""
__all__ = ["api", "synth"]
