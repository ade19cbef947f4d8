"""CPU oracle for the NF4 + double-quantized frozen linear with a LoRA side path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables, constants or
helpers with the HIP library in ``bit_nf4_quantized_dq_amd/``; the two are written
independently from the same pages, and the tests compare them.

Every function is a plain, slow, step-by-step restatement of the method as described on
the pages (cited per function by page title and section).  Where the pages are silent,
garbled or contradict one another, the reading taken is stated in the docstring.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py`` to facts
the pages or the mathematics fix independently (closed forms, other libraries' routines,
brute force, invariants, the pages' printed figures).  No function is "parity unpinned".
"""

from .qlora_oracle import (  # noqa: F401
    BLOCK1,
    BLOCK2,
    E4M3_MAX,
    nf4_codebook,
    nf4_codebook_exact,
    nearest_level,
    pack_codes,
    unpack_codes,
    e4m3_value,
    e4m3_encode,
    bf16_round_bits,
    bf16_bits_to_f32,
    quantize,
    decode_scales,
    dequantize_bf16_bits,
    dequantize_f64,
    lora_fwd,
    lora_bwd,
    quant_sizes,
    bits_per_param,
    bf16_round_f64_bits,
    merge,
    quantize_bf16,
    adamw_step,
    CODEBOOKS,
    DQ_FORMATS,
    codebook,
    e5m2_value,
    e5m2_encode,
    int8_encode,
    silu,
    mlp_fwd,
    mlp_bwd,
)
