"""CPU float64 oracle (test infrastructure only; never imported by the GPU library).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
Parity of every function here is pinned by tests/test_oracle_pins.py.
"""
from .attention import (INCLUDE_SELF, SlotRing, ar_decode, as_f64, bruteforce_joint, default_scale,
                        joint, masked_attention, mfalcon_mask, pool_write, prefill,
                        prefill_rows, rank_decode, rank_decode_rows)

from .block import LN_EPS, WEIGHT_KEYS, block_candidates, block_history, block_joint, gelu, layer_norm

__all__ = ["LN_EPS", "WEIGHT_KEYS", "block_candidates", "block_history", "block_joint", "gelu", "layer_norm", "INCLUDE_SELF", "SlotRing", "ar_decode", "as_f64", "bruteforce_joint", "default_scale", "joint",
           "masked_attention", "mfalcon_mask", "pool_write", "prefill", "prefill_rows",
           "rank_decode", "rank_decode_rows"]
