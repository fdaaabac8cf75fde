"""CPU oracle of the DSA indexer -> top-k -> sparse MLA path (test infrastructure only)."""
from .dsa_oracle import *  # noqa: F401,F403
from .dsa_oracle import (E4M3FN, NoDonorError, StaleCacheError, decode, decode_bf16, donor_map,  # noqa: F401
                         group_forward, group_stats, index_scores, index_scores_backward_selected, index_scores_loop,
                         index_scores_row,
                         parse_pattern, served_group_sizes, sparse_mla, sparse_mla_backward, sparse_mla_backward_row,
                         sparse_mla_dense_masked_row,
                         sparse_mla_row, topk, topk_row)
