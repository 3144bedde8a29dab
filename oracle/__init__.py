"""CPU fp64 oracle for frame-structured block-sparse attention.

Test infrastructure only: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path."""
from .fsattn_oracle import *  # noqa: F401,F403
from .fsattn_oracle import (MaskGeometry, live_frames, token_mask, row_mask, mask_rows,  # noqa: F401
                            plan_bruteforce, attention_ref, attention_live_ref, attention_online_ref,
                            attention_fixed_shift_ref, head_bounds_ref, row_shift_ref,
                            live_logit_stats, live_flops, partial_blocks_if_tiled,
                            rms_norm_ref, rope_ref, produce_ref, rope_tables_1d,
                            GAP_THRESHOLD_NATS)
