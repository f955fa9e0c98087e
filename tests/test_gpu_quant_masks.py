"""GPU parity of the quantized forward and backward (int8 and int4) with masks and causal.

Page "Metal Flash Attention", section "Enable In SimpleTuner": the regular and the quantized
dispatchers both take bool masks (True = attend), additive float masks, batched [B, H, Sq,
Skv] and broadcast [B, 1, 1, Skv] masks, and all-true bool masks are skipped as a fast path.
The quantized values (codes) are those of the unmasked call: masks and causal only change
which scores count.  Forward: O and LSE against the oracle run from the GPU's own codes;
backward: every gradient element against the oracle's straight-through backward."""
import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import rope_sdpa_backward_quant, rope_sdpa_forward_quant
from parity_util import check_grad, check_lse, check_out, dev, dt_name, to64

pytestmark = pytest.mark.gpu

VARIANTS = ["causal", "bool4d", "bool_bcast", "additive4d", "additive_f32_keys", "all_true"]


def _case(variant, dtype, seed, B=2, H=3, Hkv=3, S=300, D=128):
    kw = {}
    if variant == "causal":
        kw = dict(causal=True)
    elif variant == "bool4d":
        kw = dict(mask_kind="bool", mask_shape=(B, H, S, S))
    elif variant == "bool_bcast":
        kw = dict(mask_kind="bool", mask_shape=(B, 1, 1, S))
    elif variant == "additive4d":
        kw = dict(mask_kind="additive", mask_shape=(B, H, S, S))
    w = syn.random_small(B, H, S, D, dtype, seed=seed, kv_heads=Hkv, with_grad=True, **kw)
    if variant == "additive_f32_keys":
        r = np.random.default_rng(seed)
        add = np.where(r.random((B, 1, 1, S)) < 0.8, r.standard_normal((B, 1, 1, S)), -np.inf)
        w.mask, w.mask_kind = torch.from_numpy(add.astype(np.float32)), "additive"
    elif variant == "all_true":
        w.mask, w.mask_kind = torch.ones(B, 1, 1, S, dtype=torch.bool), "bool"
    return w


def _kw(w):
    return dict(mask=w.mask, mask_kind=w.mask_kind, causal=w.causal, scale=w.scale)


@pytest.mark.parametrize("mode", ["int8", "int4", "int8_prepass", "int4_prepass"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_quant_forward_masked(mode, variant):
    bits = 4 if mode.startswith("int4") else 8
    w = _case(variant, "bf16", 400 + VARIANTS.index(variant))
    d = dev()
    m = w.mask.to(d) if w.mask is not None else None
    with torch.no_grad():
        o, lse = rfa.rope_sdpa_fwd_with_lse(w.q.to(d), w.k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d), attn_mask=m,
                                            is_causal=w.causal, scale=w.scale, quantization=mode)
    qc, qs, kc, ks = (t.cpu().numpy() for t in rfa.debug_quantize_qk(w.q.to(d), w.k.to(d), w.cos.to(d),
                                                                     w.sin.to(d), bits=bits))
    torch.cuda.synchronize()
    O_ref, L_ref = rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=bits, codes=((qc, qs), (kc, ks)),
                                           workers=8, **_kw(w))
    check_out("O", to64(o), O_ref, "bf16")
    check_lse(to64(lse), L_ref, "bf16")
    # the oracle's own quantizer reaches the same codes, hence the same reference
    O_ind, _ = rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=bits, workers=8, **_kw(w))
    assert np.array_equal(O_ind, O_ref)


def test_quant_all_true_mask_is_bitwise_unmasked():
    w = _case("all_true", "bf16", 420)
    d = dev()
    with torch.no_grad():
        args = (w.q.to(d), w.k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d))
        o0, l0 = rfa.rope_sdpa_fwd_with_lse(*args, quantization="int8")
        o1, l1 = rfa.rope_sdpa_fwd_with_lse(*args, attn_mask=w.mask.to(d), quantization="int8")
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("mode", ["int8", "int4"])
@pytest.mark.parametrize("variant", ["causal", "bool4d", "additive4d"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_quant_backward_masked(mode, variant, dtype):
    bits = 4 if mode == "int4" else 8
    w = _case(variant, dtype, 430 + VARIANTS.index(variant), H=4, Hkv=2)
    d = dev()
    q, k, v = (t.to(d).detach().requires_grad_() for t in (w.q, w.k, w.v))
    m = w.mask.to(d) if w.mask is not None else None
    o = rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), attn_mask=m, is_causal=w.causal,
                                              scale=w.scale, quantization=mode)
    o.backward(w.do.to(d))
    torch.cuda.synchronize()
    O_ref, _ = rope_sdpa_forward_quant(w.q, w.k, w.v, w.cos, w.sin, bits=bits, workers=8, **_kw(w))
    check_out("O", to64(o), O_ref, dtype)
    refs = rope_sdpa_backward_quant(w.q, w.k, w.v, w.cos, w.sin, w.do, bits=bits, workers=8, **_kw(w))
    for name, g, r in zip(("dQ", "dK", "dV"), (q.grad, k.grad, v.grad), refs):
        check_grad(name, to64(g), r, dtype)
