"""GPU parity of the quantized backward (the quantized autograd path) against the oracle.

Page "Metal Flash Attention" (SimpleTuner docs): quantized training goes through a quantized
autograd entry point (sections "Requirements" and "Enable In SimpleTuner").  Reading (the
oracle's rope_sdpa_backward_quant): the gradient passes the quantizer straight through, so
the backward is the attention backward at the dequantized rotated Q and K the forward
attended with, followed by the inverse rotation.  The HIP path rebuilds those values with
the quantizer pass in its dequantizing mode and runs the 16-bit backward kernels on them."""
import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import rope_sdpa_backward_quant, rope_sdpa_forward_quant
from parity_util import check_grad, check_out, dev, dt_name, to64

pytestmark = pytest.mark.gpu


def _gpu(w, mode):
    d = dev()
    q, k, v = (t.to(d).detach().requires_grad_() for t in (w.q, w.k, w.v))
    o = rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), scale=w.scale, quantization=mode)
    o.backward(w.do.to(d))
    torch.cuda.synchronize()
    return o, q.grad, k.grad, v.grad


def _compare(w, mode):
    bits = 4 if mode.startswith("int4") else 8
    dtype = dt_name(w.q)
    o, dq, dk, dv = _gpu(w, mode)
    assert dk.shape == w.k.shape and dv.shape == w.v.shape
    O_ref, _ = rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=bits, scale=w.scale, workers=8)
    check_out("O", to64(o), O_ref, dtype)
    refs = rope_sdpa_backward_quant(w.q, w.k, w.v, w.cos, w.sin, w.do, bits=bits, scale=w.scale, workers=8)
    for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
        check_grad(name, to64(g), r, dtype)
    # the autograd forward is the no-grad quantized forward
    d = dev()
    with torch.no_grad():
        o2 = rfa.rope_scaled_dot_product_attention(w.q.to(d), w.k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d),
                                                   scale=w.scale, quantization=mode)
    assert torch.equal(o.detach(), o2)


@pytest.mark.parametrize("mode", ["int8", "int4", "int8_prepass"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("heads", [(4, 4), (4, 2)])
def test_quant_backward_small(mode, dtype, heads):
    """B=2, S=300 (ragged tail), D=128, every element of dQ, dK, dV."""
    H, Hkv = heads
    w = syn.random_small(2, H, 300, 128, dtype, seed=300 + H + Hkv, kv_heads=Hkv, with_grad=True,
                         per_sample_tables=(Hkv == 2))
    _compare(w, mode)


@pytest.mark.parametrize("mode", ["int8", "int4"])
def test_quant_backward_flux_shape(mode):
    """FLUX joint attention shape with 4 heads: B=1, H=4, S=512+4096, D=128, 3-axis RoPE."""
    w = syn.flux(batch=1, heads=4, grid=64, dtype="bf16", seed=310, with_grad=True)
    _compare(w, mode)


def test_quant_backward_counter():
    w = syn.random_small(1, 2, 64, 128, "bf16", seed=311, with_grad=True)
    rfa.rope_sdpa_reset_stats()
    _gpu(w, "int8")
    s = rfa.get_dispatch_stats()
    assert s["quantized_autograd"] == 1 and s["backward"] == 1 and s["quantized_int8"] == 1


@pytest.mark.parametrize("mode", ["int8", "int4"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("variant", ["none", "causal", "gqa"])
def test_quant_backward_d64(mode, dtype, variant):
    """D = 64 (the 32x32 backward kernels reading the dequantized Q' and K')."""
    H, Hkv = (4, 2) if variant == "gqa" else (2, 2)
    w = syn.random_small(2, H, 300, 64, dtype, seed=312 + H, kv_heads=Hkv, with_grad=True,
                         causal=(variant == "causal"))
    bits = 4 if mode == "int4" else 8
    d = dev()
    q, k, v = (t.to(d).detach().requires_grad_() for t in (w.q, w.k, w.v))
    o = rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), is_causal=w.causal,
                                              quantization=mode)
    o.backward(w.do.to(d))
    torch.cuda.synchronize()
    kw = dict(causal=w.causal, workers=8)
    O_ref, _ = rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=bits, **kw)
    check_out("O", to64(o), O_ref, dtype)
    refs = rope_sdpa_backward_quant(w.q, w.k, w.v, w.cos, w.sin, w.do, bits=bits, **kw)
    for name, g, r in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), refs):
        check_grad(name, to64(g), r, dtype)
