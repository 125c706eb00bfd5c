"""QoQ W4A8 per-group GEMM for MI355X (gfx950).

The compute path lives in the HIP library ``_lib/libqoq.so`` (C ABI declared in
``include/qoq.h``); :mod:`.qoq` is the thin ctypes binding over it and
:mod:`.workloads` holds layer shapes and seeded synthetic inputs.  Nothing is
loaded at import time.
"""

__all__ = ["qoq", "workloads"]
