"""CPU oracle of the routed-MoE routing step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or run anything here. The HIP library and its
Python binding never do; the two share no code.
"""
from .route_ref import (  # noqa: F401
    bf16_bits_to_f64,
    bf16_rne_bits,
    biased_scores,
    exclusive_offsets,
    expert_counts,
    expert_major_permutation,
    grouped_layout,
    grouped_layout_rows,
    e4m3_code,
    e4m3_value,
    mxfp8_quantize,
    balance_plan,
    group_scores,
    kept_groups,
    local_num_experts,
    pack,
    relabel,
    renormalised_weights,
    route_ref,
    route_tokens,
    router_logits_bound,
    router_logits_ref,
    sigmoid_rn32,
    sigmoid_rn32_fallback_count,
    topk_experts,
)
