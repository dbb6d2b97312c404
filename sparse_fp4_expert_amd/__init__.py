"""MI355X-native grouped 4:8 sparse-FP4 expert GEMM (libmoesq).

The compute lives in hand-written HIP kernels behind the C ABI of
include/moesq.h; `sparse_fp4_expert_amd.moesq` is the ctypes binding.
Build the library with `python -m sparse_fp4_expert_amd.build`.
"""
__all__ = ["moesq"]
