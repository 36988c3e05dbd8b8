"""MI355X (gfx950) routed MoE layer forward: sigmoid/noaux_tc or softmax top-k
router, batch-union bucketing, dequant-on-use int4/int2/bf16 SwiGLU experts,
scaled combine plus shared expert.

The compute lives in libmoe.so (HIP kernels behind the C ABI of
include/moe.h); `capi` is the thin ctypes binding with the same function names.
"""
from . import capi  # noqa: F401

__all__ = ["capi"]
