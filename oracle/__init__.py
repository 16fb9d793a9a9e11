"""fp64 CPU oracle for Sparse Query Attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package. It shares no code with the HIP path.
"""
from .sqa_oracle import (attention, attention_bwd, attention_param_count, attention_varlen, attention_bwd_varlen, block, kv_head_index,
                         layer, layer_weight_shapes, rms_norm, rope, swiglu)

__all__ = ["attention", "attention_bwd", "attention_param_count", "attention_varlen", "attention_bwd_varlen", "block", "kv_head_index",
           "layer", "layer_weight_shapes", "rms_norm", "rope", "swiglu"]
