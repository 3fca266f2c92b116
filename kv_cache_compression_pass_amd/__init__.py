"""MI355X (gfx950) KV-cache scoring and compression: Python binding of libkvc.

The product path is the C-ABI library ``libkvc.so`` (include/kvc.h) built from the HIP
sources in ``csrc/``.  This package only marshals arguments to it; importing the functions
below loads the library and fails loudly when it has not been built.
"""

from ._lib import (  # noqa: F401
    ALLOC_K_CHANNELS, ALLOC_TOPK, ALLOC_V_TOKENS, DEV_BAD_CACHE, DEV_BAD_WIDTH, DEV_NOT_SPD, EXPORTED,
    LIB_PATH, OP_ALLOCATE_BITS, OP_CHANNEL_WEIGHTS, OP_COMPRESSED_ATTEND, OP_QUANTIZE_PACK,
    OP_RIDGE_FIT, OP_ROW_LSE, OP_SCORE_TOKENS, PK_NAMES, SCORE_MAX, SCORE_SUM, load,
)
from .api import (  # noqa: F401
    KvcError, PackedCache, alloc_result_buffer, bf16_tensor, decode_alloc_result, kvc_allocate_bits,
    kvc_keep_threshold, kvc_channel_weights, kvc_compressed_attend, kvc_compressed_attend_append,
    kvc_fidelity_terms, kvc_get_device_status, kvc_pilot_budgets, kvc_packed_capacity, kvc_ridge_value_fit,
    kvc_quantize_pack, kvc_row_lse, kvc_row_lse_noalloc, kvc_score_tokens, kvc_version, kvc_workspace_size, make_desc,
    workspace,
)
