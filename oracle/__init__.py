"""CPU fp64 oracle for GVA decode. Test infrastructure only: imported by the
test suite, the package smoke check and the benchmark's CPU-baseline leg,
never by the product path."""
from .gva_oracle import *  # noqa: F401,F403
from .gva_oracle import (append_positional_keys, gqa_decode, gva_decode, gva_decode_seq,
                         gva_decode_step, gva_head_scores, gva_scalars_per_token,
                         gqa_scalars_per_token, head_group, kv_cache_bytes,
                         materialized_keys, rope, rope_thetas, round_bf16, round_storage,
                         query_projection, fold_query_projection, gva_layer_decode_step,
                         gva_decode_multi, gva_decode_multi_step, gva_prefill, gva_prefill_step)
