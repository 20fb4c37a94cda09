"""CPU oracle for the attention hot path. TEST INFRASTRUCTURE: imported only by
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``."""

from .oracle import (  # noqa: F401
    LayerKVCache,
    allowed,
    apply_rope,
    attended_keys_total,
    attention_layer_step,
    gqa_attention,
    kv_bytes,
    kv_head_of,
    mixer_layer_step,
    offset_rms_norm,
    rope_frequencies,
    yarn_ramp_bounds,
)
