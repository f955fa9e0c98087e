"""GPU parity of grouped-query / multi-query attention (K and V with Hkv < H heads) against the
oracle: forward (O, LSE) and backward (dQ at H heads; dK, dV at Hkv heads, summed over each
group), small shapes over every dtype, head dim and mask kind, and the FLUX shape with
per-sample rotation tables at full size.  Page "Metal Flash Attention", section "Fused RoPE +
SDPA": GQA inputs are rotated at the K/V head count and expanded afterwards."""
import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import (quantize_blockwise_int8, rope_rotate_f32, rope_sdpa_backward, rope_sdpa_forward,
                    rope_sdpa_forward_int8)
from parity_util import check_grad, check_lse, check_out, dev, to64

pytestmark = pytest.mark.gpu


def _dtype(t):
    return {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[t.dtype]


def _run(w, grad):
    d = dev()
    q, k, v = (t.to(d).detach().requires_grad_(grad) for t in (w.q, w.k, w.v))
    m = w.mask.to(d) if w.mask is not None else None
    if grad:
        o = rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), attn_mask=m,
                                                  is_causal=w.causal, scale=w.scale)
        o.backward(w.do.to(d))
        torch.cuda.synchronize()
        return o, None, q.grad, k.grad, v.grad
    with torch.no_grad():
        o, lse = rfa.rope_sdpa_fwd_with_lse(q, k, v, w.cos.to(d), w.sin.to(d), attn_mask=m, is_causal=w.causal,
                                            scale=w.scale)
    torch.cuda.synchronize()
    return o, lse, None, None, None


def _compare(w, grad=True):
    dt = _dtype(w.q)
    kw = dict(mask=w.mask, mask_kind=w.mask_kind, causal=w.causal, scale=w.scale, workers=8)
    O_ref, L_ref = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, **kw)
    o, lse, dq, dk, dv = _run(w, grad=False)
    check_out("O", to64(o), O_ref, dt)
    check_lse(to64(lse), L_ref, dt)
    if grad:
        o2, _, dq, dk, dv = _run(w, grad=True)
        assert torch.equal(o2, o)
        assert dk.shape == w.k.shape and dv.shape == w.v.shape
        refs = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, **kw)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs):
            check_grad(name, to64(g), r, dt)


@pytest.mark.parametrize("variant", ["none", "causal", "bool4d", "additive"])
@pytest.mark.parametrize("heads", [(4, 2), (6, 1)])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_gqa_small(dtype, D, heads, variant):
    H, Hkv = heads
    B, S = 2, 200
    kw = {}
    if variant == "causal":
        kw = dict(causal=True)
    elif variant == "bool4d":
        kw = dict(mask_kind="bool", mask_shape=(B, H, S, S))
    elif variant == "additive":
        kw = dict(mask_kind="additive", mask_shape=(1, H, S, S))
    w = syn.random_small(B, H, S, D, dtype, seed=700 + H + Hkv + D, kv_heads=Hkv, with_grad=True, **kw)
    _compare(w)


@pytest.mark.parametrize("S", [64, 130, 257])
def test_gqa_query_tile_counts(S):
    """bf16, D=128: 1 to 3 query tiles per head and ragged tails, the group loop of the dK/dV
    kernel crossing head boundaries at every tile count."""
    w = syn.random_small(1, 8, S, 128, "bf16", seed=720 + S, kv_heads=2, with_grad=True, per_sample_tables=False)
    _compare(w)


def test_gqa_int8():
    """int8 variant with K quantized at its own head count: codes bit-exact, attention against
    the oracle run from the GPU's codes."""
    w = syn.random_small(2, 6, 150, 128, "bf16", seed=730, kv_heads=2)
    d = dev()
    qc, qs, kc, ks = (t.cpu().numpy() for t in rfa.debug_quantize_qk(w.q.to(d), w.k.to(d), w.cos.to(d),
                                                                        w.sin.to(d)))
    eqc, eqs = quantize_blockwise_int8(rope_rotate_f32(w.q, w.cos, w.sin))
    ekc, eks = quantize_blockwise_int8(rope_rotate_f32(w.k, w.cos, w.sin))
    assert kc.shape == (2, 2, 150, 128)
    assert np.array_equal(qc, eqc) and np.array_equal(kc, ekc)
    assert np.array_equal(qs.view(np.uint32), eqs.view(np.uint32)) and np.array_equal(ks.view(np.uint32), eks.view(np.uint32))
    with torch.no_grad():
        o, lse = rfa.rope_sdpa_fwd_with_lse(w.q.to(d), w.k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d),
                                            quantization="int8")
    torch.cuda.synchronize()
    O_ref, L_ref = rope_sdpa_forward_int8(w.q, w.k, w.v, w.cos, w.sin, codes=((qc, qs), (kc, ks)), workers=8)
    check_out("O", to64(o), O_ref, "bf16")
    check_lse(to64(lse), L_ref, "bf16")


def test_gqa_flux_per_sample_tables_full_size():
    """FLUX shape B=2, H=24 query heads over Hkv=6 K/V heads, S=4608, D=128, per-sample 3-axis
    tables (each item's image ids shifted by its own offset): every (b, h) of O, LSE, dQ and
    every (b, kv head) of dK, dV against the oracle."""
    w = syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=740, with_grad=True, kv_heads=6,
                 per_sample_tables=True)
    assert w.cos.shape[0] == 2
    _compare(w)
