"""CPU oracle for varlen paged attention -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy (plus a pure-Python scalar version for tiny inputs) written
from the pages' definitions.  It shares no code with the HIP library and imports
nothing from it.  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
CPU-baseline leg may import it; the product path never calls it.

Modules
-------
``attention``  : the method itself (mask, page gather, masked softmax attention).
``brute``      : the same definition as nested scalar loops (independent re-derivation
                 used to pin ``attention`` on tiny inputs).
``accounting`` : closed-form counters (KV bytes per position, visible pairs, FLOPs,
                 logical vs physical KV bytes).
``kv_append``  : writing the iteration's new K/V into the paged pools (slot mapping).
``fp8``        : fp8 e4m3fn KV storage with per-token float32 scales (decode, dequantise,
                 quantise and append new rows).

Every function is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_pins.py``;
none is "parity unpinned".
"""
from .attention import (bf16_bits_to_f64, to_f64, visibility_mask, gather_kv, attend,
                        varlen_paged_attention, attention_rows)
from .accounting import (kv_bytes_per_position, visible_pairs, attention_flops,
                         logical_kv_bytes, physical_kv_bytes)
from .brute import brute_force_attention
from .kv_append import slots_for_new_rows, append_kv
from .fp8 import e4m3fn_to_f64, dequantize_pools, e4m3fn_round, quantize_rows, append_kv_fp8

__all__ = [
    "bf16_bits_to_f64", "to_f64", "visibility_mask", "gather_kv", "attend",
    "varlen_paged_attention", "attention_rows", "kv_bytes_per_position", "visible_pairs",
    "attention_flops", "logical_kv_bytes", "physical_kv_bytes", "brute_force_attention",
    "slots_for_new_rows", "append_kv", "e4m3fn_to_f64", "dequantize_pools", "e4m3fn_round", "quantize_rows",
    "append_kv_fp8",
]
