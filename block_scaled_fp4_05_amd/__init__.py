"""NVFP4 block-scaled MoE grouped GEMM for one AMD MI355X (gfx950).

The computation lives in the HIP library ``libmoe_fp4.so`` behind the C ABI of
``include/moe_fp4.h``; ``moe_fp4`` is its Python binding (marshalling only).
"""
from . import moe_fp4  # noqa: F401
from .moe_fp4 import grouped_gemm, plan, quantize, stage_bytes  # noqa: F401
