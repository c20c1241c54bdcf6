"""dequant_gemm_amd -- NF4 blockwise quantization and fused NF4-dequant GEMMs for MI355X.

The work runs in ``libnf4.so`` (hand-written HIP for gfx950, C ABI in
``include/nf4.h``); this package is its thin Python binding.  Build the library
with ``python -m dequant_gemm_amd.build``.
"""
from ._lib import (  # noqa: F401
    BLOCKSIZE, DQ_GROUP, EXPORTS, LIB_PATH, NF4Error, QTensor, QTensorStruct,
    empty_qtensor, lib, nf4_codebook, nf4_dequantize, nf4_matmul_bwd_dx, nf4_matmul_fwd,
    nf4_quantize, nf4_sizes, nf4_thresholds,
)
