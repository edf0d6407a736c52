"""CPU oracle for the Llama 2 decoder forward -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import, call or
execute anything in this package.  The product path (the HIP library and its Python
binding) never does, and shares no code with it.

See oracle/llama.py for the definitions and the passages they follow.
"""
from .llama import (  # noqa: F401
    ModelArgs, ffn_hidden_dim, kv_cache_bytes, rms_norm, rope_frequencies, rope_angles,
    apply_rope, causal_mask, softmax, attention, silu, feed_forward, Oracle,
    argmax_lowest, sample_top_p, greedy_generate, teacher_forced_logits, args_from_workload,
    workload_weights, round_bf16, round_fp16,
)
