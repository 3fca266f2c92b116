"""Plain float64 CPU oracle for the KV-cache scoring and compression path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library or its Python binding may import, call or
link this package; only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` use it.  It shares no code, headers, tables or helpers with the HIP path.

Every function here is the plainest reading of the definition it cites, computed in IEEE
float64 from the exact bf16 inputs (bf16 -> float64 widening is exact).  Sources cited:

* "KVSculpt: KV Cache Compression as Distillation" summary page, §2 (loss: output MSE and
  log-sum-exp matching terms; the closed-form ridge value solve; the pilot budget split).
* "RDKV - rate-distortion bit allocation for joint eviction and quantization of the KV
  cache" summary page, §2.1 (token weight w_t, channel weight w_c, rate-distortion
  objective), §2.2 (allocation over the widths {0,2,4,8,16} in three stages), §2.3 (packed
  zones with fused dequantisation).
* "KVzap - fast, adaptive and faithful KV cache pruning" summary page, §2.1 (KVzip+ score),
  §2.2 (scores per KV head), §2.3 (fixed-budget keep used by KVzip).

Parity pins: every function is pinned by tests under ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force or library routines; the conventions that the pages do
not fix (packed byte layout, sigma = 1, budget scope, causal alignment, K grouping axis) are
"parity unpinned" and are listed as such where they are defined.
"""

from .common import as_f64, query_positions, default_scale
from .attention import (
    row_lse,
    token_scores_sum,
    token_scores_max,
    hidden_row_norms,
    value_out_norms,
    channel_weights,
)
from .allocation import (
    LEVELS,
    step_ratios,
    step_keys,
    lagrangian_allocate,
    stage_costs,
    allocate_v_tokens,
    allocate_k_channels,
    retained_counts,
    topk_keep,
    threshold_keep,
    pilot_budgets,
)
from .quantize import quantize_group, pack_group_words, pack_cache, HDR_GLOBAL, HDR_PER_HEAD
from .fidelity import (dequantized_head, attend, full_attend, compressed_attend, compressed_attend_append,
                       fidelity_terms, fidelity_terms_per_head)
from .ridge import ridge_normal_equations, ridge_system, ridge_value_fit

__all__ = [
    "as_f64", "query_positions", "default_scale",
    "row_lse", "token_scores_sum", "token_scores_max", "hidden_row_norms", "value_out_norms",
    "channel_weights",
    "LEVELS", "step_ratios", "step_keys", "lagrangian_allocate", "stage_costs",
    "allocate_v_tokens", "allocate_k_channels", "retained_counts", "topk_keep", "threshold_keep", "pilot_budgets",
    "quantize_group", "pack_group_words", "pack_cache", "HDR_GLOBAL", "HDR_PER_HEAD",
    "dequantized_head", "attend", "full_attend", "compressed_attend", "compressed_attend_append", "fidelity_terms", "fidelity_terms_per_head",
    "ridge_normal_equations", "ridge_system", "ridge_value_fit",
]
