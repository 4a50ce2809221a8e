"""CPU oracle (test infrastructure only; see kvc_oracle's header)."""
from .kvc_oracle import (  # noqa: F401
    bf16_to_f64, default_scale, group_logits, normalizers, scores, maxpool,
    mandatory, select_head, select, gather, inverse_stability_budgets,
    compress_layer, LayerResult, logit_scores, logit_scores_int8, pooled_query, quantize_int8,
    first_visible_row, overlap_coefficient, chunk_bounds, compress_chunked,
)
from .prefill_oracle import (  # noqa: F401,E402
    to_bf16_bits, rmsnorm, rope_cos_sin, rope, attention, silu, swiglu, LayerWeights, ModelShape,
    layer_chunk, PrefillResult, prefill_layer_major,
)
