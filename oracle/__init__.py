"""CPU fp64 oracle of one decoder-layer step (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package; the product library never does.
"""
from .layer import (layer_step, layer_step_split, rmsnorm, rope, rope_cos_sin, silu,
                    swiglu_ffn, paged_attention, attention_weights, kv_append, moe_route,
                    round_to_bf16, round_to_f32, store_round, page_slots, PAGE)
