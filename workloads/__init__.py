"""Seeded synthetic workloads shared by the oracle side and the GPU side (inputs only)."""
from .configs import (DECODE_BF16, DECODE_CONFIGS, PREFILL_BF16, PREFILL_CONFIGS, TINY_FP32,
                      TRAIN_BF16, VARCHUNK_BF16, DecodeConfig, PrefillConfig)
from .synth import (ACT_NAMES, PARAM_NAMES, DecodeInputs, PrefillInputs, ProjInputs,
                    draw_chunk_lengths, make_block_inputs, make_decode, make_stack, make_output_grad, make_prefill,
                    make_projection,
                    make_ragged_prefill, torch_dtype)
