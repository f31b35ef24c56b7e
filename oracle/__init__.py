"""CPU float64 oracle (test infrastructure only; never imported by the GPU library).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
Parity of every function here is pinned by tests/test_oracle_pins.py.
"""
from .attention import (INCLUDE_SELF, SlotRing, ar_decode, as_f64, bruteforce_joint, default_scale,
                        joint, masked_attention, mfalcon_mask, pool_write, prefill,
                        prefill_rows, rank_decode, rank_decode_rows)

from .block import LN_EPS, WEIGHT_KEYS, block_candidates, block_history, block_joint, gelu, layer_norm

from .fp8 import E4M3_MAX, ar_decode_e4m3, e4m3_decode, e4m3_encode, pool_write_e4m3

__all__ = ["E4M3_MAX", "ar_decode_e4m3", "e4m3_decode", "e4m3_encode", "pool_write_e4m3", "LN_EPS", "WEIGHT_KEYS", "block_candidates", "block_history", "block_joint", "gelu", "layer_norm", "INCLUDE_SELF", "SlotRing", "ar_decode", "as_f64", "bruteforce_joint", "default_scale", "joint",
           "masked_attention", "mfalcon_mask", "pool_write", "prefill", "prefill_rows",
           "rank_decode", "rank_decode_rows"]
