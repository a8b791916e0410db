"""FP8 W8A8 block-scaled linear layers for AMD MI355X (gfx950).

The computation lives in libfp8w8a8.so (hand-written HIP kernels behind a C
ABI declared in include/fp8w8a8.h); this package is its Python binding.
"""

from ._lib import (  # noqa: F401
    LIB_PATH, SCALE_BLOCK, SCALE_ROW, SCALE_TENSOR, block_gemm, encode_f32, grouped_gemm,
    kv_cache_read, kv_cache_write, lib, linear, linear_noalloc, quant_act, quant_act_static, quant_weight_block,
    status_str, workspace_bytes,
)
