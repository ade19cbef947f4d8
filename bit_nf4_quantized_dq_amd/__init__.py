"""MI355X (gfx950) NF4 + double-quantized frozen linear with a 16-bit LoRA side path.

The compute runs in the HIP library ``libqlora_nf4.so`` (C ABI in ``include/qlora.h``);
this package only marshals arguments.  ``lib`` raises if the library is missing -- there is
no CPU fallback.
"""

from ._binding import (  # noqa: F401
    QLoRAError,
    QuantizedWeight,
    lib,
    load_library,
    nf4_codebook,
    codebook,
    CODEBOOKS,
    DQ_FORMATS,
    quantize,
    quantize_bf16,
    merge,
    adamw_step,
    dequantize,
    linear_fwd,
    linear_fwd_noalloc,
    linear_fwd_multi,
    mlp_fwd,
    mlp_bwd,
    mlp_workspace_size,
    workspace_size_multi,
    linear_bwd,
    e4m3_encode,
    quant_sizes,
    workspace_size,
    new_workspace,
    workspace_init,
    timing_enable,
    timing_read,
    KERNEL_IDS,
    OP_QUANTIZE,
    OP_FWD,
    OP_BWD,
)
