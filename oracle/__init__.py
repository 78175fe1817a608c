"""CPU oracle (test infrastructure only; see mqa_oracle's header)."""
from .mqa_oracle import (  # noqa: F401
    E4M3FN_VALUES, HEAD_DIM, ROW_BYTES, decode_bytes, decode_e4m3fn, paged_mqa_logit_at,
    paged_mqa_logits, split_kv_rows, topk, topk_row, visible_count,
)
