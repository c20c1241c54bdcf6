"""dequant_gemm_amd -- NF4 blockwise quantization and fused NF4-dequant GEMMs for MI355X.

FP4 (the E2M1 4-bit float, levels over 6) runs through the same calls: pass
``quant_type="fp4"`` to ``nf4_quantize`` (or ``empty_qtensor``).

The work runs in ``libnf4.so`` (hand-written HIP for gfx950, C ABI in
``include/nf4.h``); this package is its thin Python binding.  Build the library
with ``python -m dequant_gemm_amd.build``.

Above the C ABI: ``dequant_gemm_amd.nn`` (NF4Linear, a frozen quantized linear
layer with autograd over the fused GEMMs) and ``dequant_gemm_amd.io`` (saving
and loading quantized weights).
"""
from ._lib import (  # noqa: F401
    BLOCKSIZE, BLOCKSIZES, DQ_GROUP, EXPORTS, LIB_PATH, NF4Error, QTensor, QTensorStruct, QUANT_TYPES,
    LORA_MAX_RANK, LORA_RANK_STEP, empty_qtensor, lib, nf4_codebook, nf4_levels, nf4_dequantize, nf4_matmul_bwd_dx,
    nf4_matmul_bwd_dx_lora, nf4_matmul_fwd, nf4_matmul_fwd_lora, nf4_quantize, nf4_quantize_noalloc, nf4_sizes, nf4_thresholds,
    NOALLOC_MAX_BLOCKS, nf4_adapter_matmul,
)
from .io import load_qtensor, load_qtensors, save_qtensor, save_qtensors  # noqa: F401,E402
from .nn import NF4Linear, NF4LoraLinear, nf4_linear, quantize_linears  # noqa: F401,E402
