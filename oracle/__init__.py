"""Oracle: a plain, slow, obviously correct CPU implementation of the X-MoD sparse-depth layer.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import or call anything in this package. The HIP library never imports it, and it
imports nothing from the HIP library or its Python binding; the two share no code. The only
thing both sides consume is the seeded input module (workload.py), which draws random
tensors and holds none of the layer's arithmetic.

Arithmetic is float64 (inputs are exact bf16 values), except where the pages' method turns a
floating-point value into an integer decision: the router logit is rounded once to fp32 and
the top-k selection is taken on fp32 values, the precision the kernels decide in. The carried
bias is fp32, updated with fp32 adds.

Parity pins (tests/test_oracle_pins.py) tie every function here to something other than
itself: printed numbers of the pages, closed forms, brute force on tiny inputs, and special
cases that reduce to a textbook definition.
"""
from .layer import (router_logits, topk_select, sigmoid, rmsnorm, causal_attention, silu,
                    swiglu_ffn, sparse_layer, dense_layer, threshold_select,
                    sparse_layer_threshold, mask_agreement, differing_selected_share,
                    qk_head_norm, rope, attention_layer, routed_ffn_layer,
                    sparse_layer_fullkv)
from .stack import (stack_layer_kinds, physical_layers, active_equivalent_layers, total_params,
                    active_params, layer_params, flops_per_token_pages_convention, block_forward,
                    coverage, adjacent_jaccard, coverage_independent_reference,
                    jaccard_independent_reference)
from .backward import (rmsnorm_grad, causal_attention_grad, silu_grad, route_bce,
                       route_bce_grad, sparse_layer_grad)
from .numerics import bf16_to_f64, round_to_bf16, f64_to_bf16_bits
