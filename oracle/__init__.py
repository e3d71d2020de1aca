"""Float64 CPU oracle (test infrastructure only; see spot_oracle)."""
from .spot_oracle import *  # noqa: F401,F403
from .spot_oracle import (attend_decode, attend_prefill, decode, indexer_scores, key_importance,
                          key_permutation, meanpool_scores, pool_blocks, prefill, select_decode,
                          select_prefill, topp_detail, topp_keep)
