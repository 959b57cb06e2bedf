"""MI355X-native Kaczmarz Linear Attention (KLA) operator.

``chunk_fwd`` (chunkwise prefill) and ``decode_step`` (one recurrent step)
call the hand-written gfx950 HIP kernels in libkla.so through its C ABI
(include/kla.h).  The library is loaded on first use; importing this package
does not touch the GPU.
"""

__all__ = ["chunk_fwd", "decode_step"]


def chunk_fwd(*args, **kwargs):
    from .kla import chunk_fwd as _f
    return _f(*args, **kwargs)


def decode_step(*args, **kwargs):
    from .kla import decode_step as _f
    return _f(*args, **kwargs)
