"""MI355X (gfx950) kernels for the online hot path of rotational W4A4
quantisation: randomized Hadamard rotation + per-token INT4, the offline
weight fold, the W4A4 GEMM and the per-head KV-cache rotation.

The compute lives in librq.so (HIP, C ABI in include/rq.h); this package only
binds it.  ``datagen`` holds the seeded synthetic input generators.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    RQError,
    decode_attention,
    decode_attention_workspace,
    fold_weights,
    fold_weights_grouped,
    fwht_quant,
    fwht_quant8,
    fwht_quant_asym,
    kv_rotate_quant,
    linear_decode,
    linear_decode_noalloc,
    linear_decode_w4a8,
    linear_decode_workspace,
    quantize_groups,
    load_library,
    status_string,
    version,
    weight_code_sums,
    w4a4_gemm,
    pack_f6,
    w4a4_gemm_f6,
    w4a4_gemm_asym,
    w4a4_gemm_grouped,
    w4a4_linear,
    w4a4_linear_asym,
    w4a8_gemm,
    w4a8_linear,
)
from .build import LIB_PATH  # noqa: F401
