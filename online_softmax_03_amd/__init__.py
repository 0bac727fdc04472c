"""MI355X-native attention forward with online softmax.

The computation lives in libfa.so (hand-written gfx950 HIP kernels behind the
C ABI of include/fa.h). `capi` is the ctypes binding with the header's names;
`attention.attention_fwd` is the torch-tensor front end; `workloads` draws the
seeded synthetic inputs.
"""
from . import capi  # noqa: F401

__all__ = ["capi", "attention_fwd"]


def attention_fwd(*args, **kwargs):
    from .attention import attention_fwd as f
    return f(*args, **kwargs)
