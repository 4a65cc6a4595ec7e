"""CPU oracle for the quantized linear layer -- TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, float64 reference that the HIP path is checked
against. Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``dequant_matmul_gptq_amd``) never imports, calls or links anything here, and
nothing here imports the product path: the two share no code.

Every function follows the pages' description of the method:

* GPTQ group-wise weights, one scale and one zero point per group of rows
  (ExLlamaV2 artifact page, GPTQ paragraph; ExLlamaV2 README, "EXL2 quantization").
* EXL2 mixed bit widths {2,3,4,5,6,8} per group, rows remapped by act-order
  (ExLlamaV2 blog, "The Investigation", Finding 3; README, "EXL2 quantization").
* Fused dequantize-and-multiply with float32 accumulation and a float16 output
  (ExLlamaV2 blog, "How the Fused CUDA Kernel Works").
* The fused output epilogue: bias, activation, residual (ExLlamaV2 artifact
  page, GPTQ paragraph: kernels fuse scaling, addition and activation).
* The on-the-fly LoRA update, joined to the epilogue as an addend (ExLlamaV2
  artifact page, LoRA adapters).
* EXL2 two-level scales: 4-bit scale codes times a per-output maximum scale
  (ExLlamaV2 blog, "How the EXL2 Quantization Pipeline Works Under the Hood",
  Step 3, and "How the Fused CUDA Kernel Works"). The value of a scale code is
  a reading of this package (parity unpinned).
* The Q4/Q6/Q8 KV-cache codec (ExLlamaV2 blog, comparison table and "How to
  Use Effectively", Step 2): a block format of this package's own
  (``kv_oracle``), since the pages give only the modes and their savings.
"""

from .qlinear_oracle import (  # noqa: F401
    BITS_SUPPORTED,
    GROUP_SIZES_SUPPORTED,
    block_field_map,
    group_word_offsets,
    packed_rows,
    pack,
    unpack,
    panel_layout,
    panel_unlayout,
    PANEL,
    zero_points,
    dequant,
    dequant_fp16,
    qlinear,
    qlinear_gidx,
    qlinear_bruteforce,
    ACT_NONE,
    ACT_SILU,
    silu,
    apply_epilogue,
    lora_delta,
    QSCALE_CODES_PER_WORD,
    qscale_pack,
    qscale_unpack,
    two_level_scales,
    dequant_qscale,
    dequant_qscale_fp16,
    qlinear_qscale,
)
from .kv_oracle import (  # noqa: F401
    KV_BITS,
    KV_GROUPS,
    kv_scales,
    kv_codes,
    kv_pack,
    kv_unpack,
    kv_quantize,
    kv_dequantize,
    kv_bytes_per_element,
)
