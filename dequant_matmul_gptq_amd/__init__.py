"""MI355X (gfx950) quantized linear layer: GPTQ 4-bit and EXL2 mixed-bit codes
unpacked, scaled and fused into the matmul against float16 activations.

The compute lives in libqlinear.so (hand-written HIP, C ABI in
include/qlinear.h); this package is its thin Python binding. PyTorch provides
device memory and streams only.
"""

from ._lib import (  # noqa: F401
    ACT_NONE,
    ACT_SILU,
    EXPORTS,
    GEMV_MAX_M,
    LIB_PATH,
    MAX_GROUP,
    MAX_RUNS,
    Layout,
    QlinearError,
    dequant,
    group_order,
    lib,
    lora_delta,
    lora_workspace_bytes,
    pack_weights,
    qgemm,
    qgemm_workspace_bytes,
    qgemv,
    qgemv_grouped,
    qgemv_noalloc,
    NOALLOC_MAX_K,
    qgemv_workspace,
    qgemv_workspace_bytes,
    reorder_groups,
    status_string,
    unpack,
    pack_qscale,
    dequant_qscale,
    qgemv_qscale,
    qgemm_qscale,
    kv_quant,
    kv_dequant,
)
