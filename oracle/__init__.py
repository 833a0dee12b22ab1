"""CPU oracle (float64, numpy) for paged KV decode attention and the KV write (bf16 or fp16
inputs).

Test infrastructure only: imported by the tests, the smoke check and the benchmark's CPU
baseline leg, never by the HIP product path.
"""
from .oracle import (bf16_bits_to_f64, f16_bits_to_f64, decode_bits, f64_to_f16_bits,
                     round_output, INPUT_DTYPES, kv_write, kv_head_for, gather_dense, attend_one,
                     effective_scale, decode_attention, decode_step, prefill_attention,
                     partial_stats,
                     merge_partials, split_attend_one, rope_pairs, rope_angles, rope_rotate,
                     f64_to_bf16_bits, kv_write_rope)

__all__ = ["bf16_bits_to_f64", "f16_bits_to_f64", "decode_bits", "f64_to_f16_bits",
           "round_output", "INPUT_DTYPES", "kv_write", "kv_head_for", "gather_dense", "attend_one",
           "effective_scale", "decode_attention", "decode_step", "prefill_attention", "partial_stats",
           "merge_partials", "split_attend_one", "rope_pairs", "rope_angles", "rope_rotate",
           "f64_to_bf16_bits", "kv_write_rope"]
