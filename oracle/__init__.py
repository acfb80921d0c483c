"""CPU oracle of the compressor hot path (test infrastructure).

Plain, slow, float64 NumPy implementations of what the GPU path computes, used
only by tests/, the smoke check and the benchmark's CPU-baseline leg. It shares
no code with the HIP library and never imports it.
"""
from .compressor import (Config, State, Weights, add_bias, decode_step, entry_candidates,
                         plain_projection, pool, prefill, project, rms_norm_bf16, softmax_weights)
from .formats import (AMAX_FLOOR, E2M1_VALUES, E4M3FN_VALUES, E8M0_AMAX_FLOOR, FP4_BLOCK, LATENT_BLOCK,
                      bf16_bits, bf16_from_bits, bf16_round, e2m1_decode, e2m1_encode, e4m3fn_decode,
                      e4m3fn_encode, fp4_quant_e4m3, fp4_quant_e8m0, fp4_unpack, pow2_ceil_exponent)
from .rope import apply_rope, rope_table, yarn_inv_freq
