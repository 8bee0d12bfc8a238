"""FP8 (OCP e4m3) MoE prefill hot path for AMD Instinct MI355X (gfx950).

The computation lives in ``libfp8moe.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fp8moe.h``). This package is its thin binding plus the composition
of the calls into an MoE layer, a W8A8 projection and the depth stack around them. Importing it fails if the library
has not been built (``python fp8_moe_prefill_amd/build.py``).
"""

from ._lib import (  # noqa: F401
    DTYPE_BF16, DTYPE_F32, EPI_STORE, EPI_SWIGLU_QUANT, GROUP, QUANT_ROW, Fp8MoeError,
    LIB_PATH, abi_version, bf16_gemm, causal_attention, fp8_dense_gemm, fp8_dense_gemm_rowwise,
    fp8_block_gemm, fp8_grouped_expert_gemm, fp8_quant_weight_block128, mxfp4_grouped_expert_gemm,
    mxfp4_quant_act, fp8_quant_act, moe_route_permute, moe_route_permute_noalloc,
    moe_unpermute_combine, pack_expert_bank, quant_route, rmsnorm, workspace_bytes,
)
from .layer import ExpertBank, MoELayerRunner, moe_layer, quantize_weight, w8a8_linear  # noqa: F401
from .stack import DepthStack, StackRunner  # noqa: F401
