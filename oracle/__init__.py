"""CPU oracle (test infrastructure only; see sparse_attn_oracle's header)."""
from .sparse_attn_oracle import *  # noqa: F401,F403
from .sparse_attn_oracle import (page_summary, page_scores, select_pages, forced_pages,
                                 rank_candidates, sparse_decode, softmax_attend, gather_tokens,
                                 row_pages, split_ranges, lse_merge, gqa_union_block_table,
                                 block_sparse_prefill, n_pages_of, valid_tokens, PER_KV_HEAD,
                                 PER_Q_HEAD)
