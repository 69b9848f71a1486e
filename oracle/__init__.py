"""Float64 CPU oracle of the MoE layer -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does.
"""
from .moe_oracle import (  # noqa: F401
    OracleLayer, brute_force_topk, combine, decode_bf16, decode_f16, decode_f32,
    decode_q4, decode_stored, exact_logit, exact_logits_fraction, expert_swiglu,
    gamma, logits_with_bound, moe_given, moe_tokens, route_token, select_topk,
    silu, softmax_gates,
)
from .from_spec import decode_act, layer_from_spec, tokens_f64  # noqa: F401
