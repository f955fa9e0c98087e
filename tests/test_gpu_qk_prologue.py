"""GPU parity of the forward's Q/K prologue against the oracle: RMSNorm of Q and K over the
head dimension before the rotation, and fp32 Q/K beside a 16-bit V (the layout autocast hands
flux-style attention: diffusers issue "Flux-family attention: flash-attn and other backends
fail in an autocast context", sections "Describe the bug" and "Root cause, in order").  The
kernel reads Q and K in their own dtype, normalizes and rotates in fp32 and rounds Q' and K'
to V's dtype for the matrix products, so O is held to V's dtype's bound."""
import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import rope_sdpa_forward
from parity_util import check_lse, check_out, dev, dt_name, to64

pytestmark = pytest.mark.gpu


def _gpu(w, q, k, norm, lse=True):
    d = dev()
    kw = dict(attn_mask=w.mask.to(d) if w.mask is not None else None, is_causal=w.causal, scale=w.scale)
    if norm is not None:
        kw.update(q_norm_weight=norm[0].to(d), k_norm_weight=norm[1].to(d), norm_eps=norm[2])
    with torch.no_grad():
        if lse:
            o, l = rfa.rope_sdpa_fwd_with_lse(q.to(d), k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d), **kw)
        else:
            o, l = rfa.rope_scaled_dot_product_attention(q.to(d), k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d),
                                                         **kw), None
    torch.cuda.synchronize()
    assert o.dtype == w.v.dtype
    return o, l


def _ref(w, q, k, norm, rows=None, pairs=None):
    kw = dict(mask=w.mask, mask_kind=w.mask_kind, causal=w.causal, scale=w.scale, rows=rows, pairs=pairs,
              workers=8)
    if norm is not None:
        kw.update(q_norm_weight=norm[0], k_norm_weight=norm[1], norm_eps=norm[2])
    return rope_sdpa_forward(q, k, w.v, w.cos, w.sin, **kw)


def _case(vdtype, qk_f32, D, variant, seed, heads=(2, 2), S=300, std=1.0):
    B, (H, Hkv) = 2, heads
    kw = {}
    if variant == "causal":
        kw = dict(causal=True)
    elif variant == "bool4d":
        kw = dict(mask_kind="bool", mask_shape=(B, H, S, S))
    elif variant == "bool_keys":
        kw = dict(mask_kind="bool", mask_shape=(B, 1, 1, S))
    w = syn.random_small(B, H, S, D, vdtype, seed=seed, kv_heads=Hkv, **kw)
    if qk_f32:  # fp32 Q and K with values off the 16-bit grid
        shape_q, shape_k = tuple(w.q.shape), tuple(w.k.shape)
        q = syn.normal(seed, syn.STREAM_Q, shape_q, "f32", std)
        k = syn.normal(seed, syn.STREAM_K, shape_k, "f32", std)
    else:
        q, k = w.q, w.k
    return w, q, k


@pytest.mark.parametrize("variant", ["none", "causal", "bool4d", "bool_keys"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mode", ["f32qk_bf16", "f32qk_f16", "f32qk_bf16_norm", "bf16_norm", "f16_norm",
                                  "f32_norm"])
def test_prologue_small(mode, D, variant):
    """B=2, H=2, S=300 (three query tiles, a ragged tail) over every prologue, dtype, head dim
    and mask kind the prologue accepts: every element of O and LSE against the oracle."""
    vdt = {"f32qk_bf16": "bf16", "f32qk_f16": "f16", "f32qk_bf16_norm": "bf16", "bf16_norm": "bf16",
           "f16_norm": "f16", "f32_norm": "f32"}[mode]
    qk_f32 = mode.startswith("f32qk")
    seed = 40 + D + 7 * ["none", "causal", "bool4d", "bool_keys"].index(variant)
    w, q, k = _case(vdt, qk_f32, D, variant, seed, std=3.0 if "norm" in mode else 1.0)
    norm = (*syn.norm_weights(seed, D), 1e-6) if "norm" in mode else None
    o, lse = _gpu(w, q, k, norm)
    O_ref, L_ref = _ref(w, q, k, norm)
    check_out("O", to64(o), O_ref, vdt)
    check_lse(to64(lse), L_ref, vdt)


def test_prologue_gqa_per_sample_tables():
    """fp32 Q/K with RMSNorm, 6 query heads over 2 K/V heads, per-sample tables."""
    seed = 51
    w = syn.random_small(2, 6, 200, 128, "bf16", seed=seed, kv_heads=2, per_sample_tables=True)
    q = syn.normal(seed, syn.STREAM_Q, tuple(w.q.shape), "f32", 3.0)
    k = syn.normal(seed, syn.STREAM_K, tuple(w.k.shape), "f32", 3.0)
    norm = (*syn.norm_weights(seed, 128), 1e-5)
    o, lse = _gpu(w, q, k, norm)
    O_ref, L_ref = _ref(w, q, k, norm)
    check_out("O", to64(o), O_ref, "bf16")
    check_lse(to64(lse), L_ref, "bf16")


def test_fp32_qk_on_the_bf16_grid_is_bitwise_the_bf16_call():
    """fp32 Q/K holding bf16 values go through the same rotation and roundings as the bf16
    call: O and LSE equal it bit for bit (FLUX shape, 4 heads, text padding mask)."""
    w = syn.flux(batch=1, heads=4, grid=32, dtype="bf16", seed=52)  # S = 512 + 1024
    o0, l0 = _gpu(w, w.q, w.k, None)
    o1, l1 = _gpu(w, w.q.float(), w.k.float(), None)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_norm_eps_and_zero_rows():
    """norm_eps reaches the kernel (a large eps changes the result as the oracle says), and an
    all-zero Q or K row normalizes to zero instead of NaN."""
    seed = 53
    w, q, k = _case("bf16", True, 128, "none", seed, std=0.05)
    q[0, 0, 5] = 0.0
    k[1, 1, 7] = 0.0
    for eps in (1e-6, 1e-2):
        norm = (*syn.norm_weights(seed, 128), eps)
        o, lse = _gpu(w, q, k, norm)
        O_ref, L_ref = _ref(w, q, k, norm)
        check_out("O", to64(o), O_ref, "bf16")
        check_lse(to64(lse), L_ref, "bf16")


@pytest.mark.parametrize("variant", ["none", "bool_padding"])
def test_flux_fp32_qk_rmsnorm_full_size(variant):
    """The FLUX shape as autocast runs it: B=1 (B=2 with the text padding mask), H=24,
    S=512+4096, D=128, fp32 Q/K after RMSNorm in the kernel, bf16 V and O.  Every head runs;
    rows 0..S-1 step 37 plus the last of every head are checked against the oracle."""
    B = 2 if variant == "bool_padding" else 1
    seed = 54
    w = syn.flux(batch=B, heads=24, grid=64, dtype="bf16", seed=seed)
    S = w.q.shape[2]
    q = syn.normal(seed, syn.STREAM_Q, tuple(w.q.shape), "f32", 4.0)
    k = syn.normal(seed, syn.STREAM_K, tuple(w.k.shape), "f32", 4.0)
    if variant == "bool_padding":
        w.mask, w.mask_kind = syn.key_padding_mask(syn.key_padding_lengths(seed, B), 512, S), "bool"
    norm = (*syn.norm_weights(seed, 128), 1e-6)
    o, lse = _gpu(w, q, k, norm)
    rows = np.unique(np.concatenate([np.arange(0, S, 37), [S - 1]]))
    O_ref, L_ref = _ref(w, q, k, norm, rows=rows)
    o64 = to64(o)[:, :, rows]
    check_out("O", o64, O_ref.reshape(o64.shape), "bf16")
    check_lse(to64(lse)[:, :, rows], L_ref.reshape(o64.shape[:3]), "bf16")


def test_prologue_is_forward_only():
    """No gradient through the prologue, no additive mask, no int8 with it."""
    seed = 55
    w, q, k = _case("bf16", True, 64, "none", seed)
    d = dev()
    qd = q.to(d).requires_grad_(True)
    with pytest.raises(rfa.RopeSdpaError):
        rfa.rope_scaled_dot_product_attention(qd, k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d))
    add = torch.zeros(1, 1, 1, q.shape[2], dtype=torch.bfloat16, device=d)
    with pytest.raises(rfa.RopeSdpaError):
        rfa.rope_scaled_dot_product_attention(q.to(d), k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d),
                                              attn_mask=add)
    with pytest.raises(rfa.RopeSdpaError):
        rfa.rope_scaled_dot_product_attention(q.to(d), k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d),
                                              quantization="int8")
    qn, kn = syn.norm_weights(seed, 64)
    with pytest.raises(rfa.RopeSdpaError):
        rfa.rope_scaled_dot_product_attention(w.q.to(d), w.k.to(d), w.v.to(d), w.cos.to(d), w.sin.to(d),
                                              q_norm_weight=qn.to(d), k_norm_weight=kn.to(d),
                                              quantization="int8_prepass")
