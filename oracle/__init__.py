"""CPU oracle of the MTLA hot path -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product path never does.
"""
from .mtla import *  # noqa: F401,F403
from .mtla import (slot_of, n_slots, is_group_final, visible, mask_matrix, sigmoid,  # noqa: F401
                   position_branch, latent, merge_weight, frame_update, with_position_table,
                   gated_latents, intermediate_states, compressed_cache, absorbed_queries,
                   softmax_rows, output_projection, prefill, attend_cache, merge_append,
                   decode_step, decode_sequence, mha_unabsorbed, prefill_predownsampled)
