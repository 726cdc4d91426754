"""CPU oracle (test infrastructure only; see moe_oracle's header)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (accept, as_f64, bf16_bits_to_f64, draft_inputs, draft_step, expert_ffn, final_norm,
                         gate_weights,
                         greedy_decode, lm_head_argmax, moe_layer, rms_norm, round_bf16, router_logits,
                         select_topk, silu, speculative_decode, verify_step)
