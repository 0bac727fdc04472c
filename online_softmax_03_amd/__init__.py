"""MI355X-native attention forward with online softmax.

The computation lives in libfa.so (hand-written gfx950 HIP kernels behind the
C ABI of include/fa.h). `capi` is the ctypes binding with the header's names;
`attention.attention_fwd` is the torch-tensor front end of the attention
forward, `softmax.softmax_rows` that of the standalone row softmax;
`workloads` draws the seeded synthetic inputs.
"""
from . import capi  # noqa: F401

__all__ = ["capi", "attention_fwd", "attention_fwd_fp8", "attention_bwd", "softmax_rows"]


def attention_fwd(*args, **kwargs):
    from .attention import attention_fwd as f
    return f(*args, **kwargs)


def attention_fwd_fp8(*args, **kwargs):
    from .attention import attention_fwd_fp8 as f
    return f(*args, **kwargs)


def attention_bwd(*args, **kwargs):
    from .attention import attention_bwd as f
    return f(*args, **kwargs)


def softmax_rows(*args, **kwargs):
    from .softmax import softmax_rows as f
    return f(*args, **kwargs)
