"""CPU oracle of the QSA indexer hot path.  Test infrastructure only: the
product library never imports it (see qsa_oracle's header)."""
from .qsa_oracle import *  # noqa: F401,F403
from .qsa_oracle import (bf16_from_f32, f32_from_bf16, rb, rope_inv_freq, rope_cos_sin,
                         rope_partial, rms_norm_1pw, block_mean, pool_keys, prep_queries,
                         score_rows, select_mask, select_mask_row, kept_blocks,
                         visible_blocks, check_budget, index_mask, gather_kv, SCORE_SCALE,
                         STATUS_BAD_INDEX)
