"""CPU oracle (float64 NumPy) of the Attamba KV-SSM forward, attention, decode and backward.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU
baseline; never by the product path.
"""
from .attamba_oracle import (TEST, TRAIN, DecodeSeq, boundary_states, chunk_attention,
                             chunk_attention_backward, masked_attention_backward,
                             selective_scan_backward,
                             decode_state_from_prefix, decode_step, dense_mask,
                             is_chunk_end_at, is_chunk_start_at, kvssm_forward, linear,
                             masked_attention, segment, selective_scan, softplus,
                             uniform_chunk_starts, silu, chunk_causal_conv, ssm_block_scan,
                             round_to_bf16, stack_forward)
