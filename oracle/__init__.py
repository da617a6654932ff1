"""CPU oracle (test infrastructure only; see rotattn_oracle's header)."""
from .rotattn_oracle import *  # noqa: F401,F403
from .rotattn_oracle import (L_BLOCK, P_LEVELS, ROPE_BASE, all_rope_tables, apply_rope,  # noqa: F401
                             ceil_f32, forward_head, fp16_attention, int4_attention, kappa,
                             nearest_f32, partition_offsets, pcode, pcode_thresholds,
                             prepare_head, qkv_projection, quantize_blocks, rope_tables,
                             rotate, softmax_attention, split_qkv, token_coords)
