"""CPU oracle (test infrastructure only; see mqa_oracle's header)."""
from .mqa_oracle import (  # noqa: F401
    E4M3FN_MAX, E4M3FN_VALUES, HEAD_DIM, ROW_BYTES, block_size_of, decode_bytes, decode_e4m3fn,
    encode_e4m3fn, mqa_logits, paged_mqa_logit_at, paged_mqa_logits, quantize_k_row, split_kv_rows, token_rows, topk,
    topk_row, visible_count, write_k_cache,
)
from .sparse_mla_oracle import (  # noqa: F401
    MLA_HEADS, MLA_KV_DIM, MLA_V_DIM, mla_block_size_of, mla_rows_of, sparse_mla_decode, sparse_mla_error_bound,
)
