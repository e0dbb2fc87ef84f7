"""DeepSeek Sparse Attention (DSA) forward path for MI355X (gfx950).

The work runs in libdsa.so (hand-written HIP kernels behind a C ABI, see
include/dsa.h); ``binding`` marshals torch tensors into it.  Importing
``sparse_long_context_relu_amd.binding`` fails loudly if the library has not
been built (``python -m sparse_long_context_relu_amd.build``).
"""
__all__ = ["binding", "build"]
