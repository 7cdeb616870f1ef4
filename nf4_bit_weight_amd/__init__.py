"""MI355X (gfx950) fused NF4 dequantise-and-multiply.

The compute lives in libnf4.so (hand-written HIP kernels behind the C ABI of
include/nf4.h).  This package is its Python binding: `api` marshals tensors to
the C entry points, `autograd` wraps them as checkpoint-visible Functions.
Importing the package does not load the library; the first call does, and it
raises if the library has not been built.
"""

from .api import (NF4Weight, nf4_dequantize, nf4_grouped_matmul_bwd_input,  # noqa: F401
                  nf4_grouped_matmul_fwd, nf4_matmul_bwd_input, nf4_matmul_fwd,
                  nf4_path_counts, nf4_quantize, nf4_reset_path_counts, nf4_workspace_bytes)
from .autograd import NF4GroupedMatMul, NF4MatMul, nf4_grouped_linear, nf4_linear  # noqa: F401
