"""CPU float64 oracle for fused rotary position embedding + scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package: only
the tests, the smoke check and the bench's CPU-baseline leg call it.  It shares no
code with the HIP kernels or their host library and never reads their outputs.

What it computes is the plain definition on the page "Metal Flash Attention"
(SimpleTuner docs), section "Fused RoPE + SDPA":

    O = softmax(scale * R(Q) R(K)^T + M) V,   scale defaults to 1/sqrt(D)

with R the interleaved-pair rotation driven by caller-supplied cos/sin tables, masks
as in the section "Enable In SimpleTuner" (bool True = attend, additive float,
broadcast up to 4-D), a causal mode, grouped-query attention (K/V with fewer heads,
rotated at their own head count and expanded), and gradients with respect to the
unrotated Q and K (the inverse rotation applied to dQ/dK).  The blockwise int8 and int4
variants follow the quantizer step by step and then apply the same definition to the
dequantized rotated Q and K; their backward passes the gradient straight through the
quantizer (the reading stated at rope_sdpa_backward_quant).

Pins: every function here is checked in tests/test_oracle_*.py against something
other than itself (naive textbook softmax, torch float64 SDPA as a library routine,
finite differences, closed forms, invariants of the rotation).  No function is
"parity unpinned".
"""
from .rope_sdpa_ref import (  # noqa: F401
    rope_rotate,
    rope_rotate_vjp,
    mask_to_additive,
    attention_forward,
    attention_backward,
    rope_sdpa_forward,
    rope_sdpa_backward,
    rope_rotate_f32,
    quantize_blockwise,
    quantize_blockwise_int8,
    quantize_blockwise_int4,
    quantized_qk,
    rope_sdpa_forward_int8,
    rope_sdpa_forward_quant,
    rope_sdpa_backward_quant,
    expand_kv,
    reduce_kv,
    rms_norm,
)
