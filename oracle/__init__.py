"""CPU oracle for MXFP8 quantization + block-scaled grouped GEMM.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the HIP library or its binding.  Plain numpy, fp64.
"""

from .mxfp8 import (  # noqa: F401
    bf16_to_f64, e4m3_decode, e4m3_encode, e8m0_from_amax, e8m0_value, quantize_blocks,
    quantize_rowwise, quantize_colwise, quantize_32x32, dequant_rowwise, dequant_32x32,
    grouped_gemm_mx, grouped_mm_fwd, grouped_mm_dgrad, grouped_mm_wgrad, group_bounds,
)
from .compare import r1_check, rne_bf16, ulp_bf16  # noqa: F401
from .route import (  # noqa: F401
    route_groups, gather_rows, scatter_rows, routed_fwd, routed_dgrad, routed_wgrad, topk_sum_rows,
)
