"""MiniMax Sparse Attention (MSA) forward path for AMD MI355X (gfx950).

The kernels and the C ABI live in libmsa.so (sources under csrc/, header in
include/msa.h); `block_sparse_long_score_amd.msa` is the thin Python binding.
Importing the package does not load the library; the first call does.
"""

from .inputs import WORKLOADS, Shape, make_inputs  # noqa: F401
