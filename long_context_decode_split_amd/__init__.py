"""helixdecode: KV-parallel (sequence-split) decode attention for MI355X.

The compute path lives in the HIP library ``libhelixdecode.so`` (C ABI,
declared in ``include/helixdecode.h``); ``api`` is a thin ctypes binding over
it that only marshals torch tensors into pointers.  Importing this package
does not load the library; the first call into ``api`` does, and fails
loudly when it has not been built.
"""

__all__ = ["api", "configs", "roofline", "synth"]
