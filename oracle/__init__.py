"""Float64 CPU oracle for large-head-dim fused attention.

TEST INFRASTRUCTURE: plain, slow, obviously correct numpy code that the HIP
path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path
(``head_dim_attention_flash_amd``) never does, and the two share no code.

Pins (tests that tie this oracle to something other than itself) live in
``tests/test_oracle_*.py``: a literal triple-loop definition with math.fsum,
torch's float64 CPU scaled_dot_product_attention and autograd, central finite
differences, closed forms (Q = 0, Nkv = 1, causal row 0, constant V) and
structural invariants (masking = deleting keys, GQA = repeat_interleave,
row independence, key permutation, backward sum rules).
"""
from .attention import (attn_bwd, attn_fwd, attn_probs, dropout_keep, dropout_threshold,
                        philox4x32_10, to_f64)

__all__ = ["attn_fwd", "attn_bwd", "attn_probs", "to_f64", "philox4x32_10", "dropout_threshold",
           "dropout_keep"]
