"""CPU oracle of the Library-of-Layers routed core (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import anything under ``oracle/``.  The product
path (``runtime_routed_transformer_amd``) never does.
"""
from .lol_oracle import (  # noqa: F401
    OracleResult, Route, BlockParams, window_offset, window_ids, partition,
    window_means, router_inputs, route, rms_norm, rope, window_causal_attention,
    silu, gelu_erf, expert_block, expert_params, forward, forward_docs,
    DecodeState, decode_state, block_step, decode,
    embed, causal_stack, lm_head, FullResult, full_forward,
)
