"""GPU parity of the eager path's two halves and of the pages' chain benchmark.

  * rope_sdpa_rotate (the eager rotation pass) against the oracle's fp32 rotation, bit for
    bit after rounding to the operand's dtype (both round every product and sum to fp32);
  * plain attention (no tables) against the oracle with identity tables;
  * the 12-layer chain at the Z-Image shape (1, 30, 4128, 128) bf16, page "Metal Flash
    Attention", section "Fused RoPE + SDPA": fused (rope_scaled_dot_product_attention per
    layer) and eager (rotation pass on the query and the keys, then plain attention), every
    layer of both against the oracle run from that layer's GPU input.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import rope_rotate_f32, rope_sdpa_forward
from parity_util import check_lse, check_out, dev, to64

pytestmark = pytest.mark.gpu

_T = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("layout", ["contiguous", "bshd_view", "in_place", "per_sample"])
def test_rotate_matches_oracle_bitwise(dtype, D, layout):
    w = syn.random_small(2, 3, 77, D, dtype, seed=800 + D, per_sample_tables=(layout == "per_sample"))
    d = dev()
    if layout == "bshd_view":
        x = w.q.transpose(1, 2).contiguous().to(d).transpose(1, 2)
        out = torch.empty(w.q.shape[0], w.q.shape[2], w.q.shape[1], D, dtype=w.q.dtype, device=d).transpose(1, 2)
        got = rfa.rope_rotate(x, w.cos.to(d), w.sin.to(d), out=out)
    elif layout == "in_place":
        x = w.q.to(d)
        got = rfa.rope_rotate(x, w.cos.to(d), w.sin.to(d), out=x)
    else:
        got = rfa.rope_rotate(w.q.to(d), w.cos.to(d), w.sin.to(d))
    torch.cuda.synchronize()
    ref = torch.from_numpy(rope_rotate_f32(w.q, w.cos, w.sin)).to(_T[dtype])
    assert torch.equal(got.cpu(), ref)


@pytest.mark.parametrize("variant", ["none", "causal", "bool_bcast", "additive"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_plain_attention_matches_oracle(dtype, D, variant):
    B, H, S = 2, 2, 300
    kw = {}
    if variant == "causal":
        kw = dict(causal=True)
    elif variant == "bool_bcast":
        kw = dict(mask_kind="bool", mask_shape=(B, 1, 1, S))
    elif variant == "additive":
        kw = dict(mask_kind="additive", mask_shape=(1, H, S, S))
    w = syn.random_small(B, H, S, D, dtype, seed=810 + D, **kw)
    d = dev()
    with torch.no_grad():
        o = rfa.scaled_dot_product_attention(w.q.to(d), w.k.to(d), w.v.to(d),
                                             attn_mask=w.mask.to(d) if w.mask is not None else None,
                                             is_causal=w.causal)
    torch.cuda.synchronize()
    ident_c, ident_s = torch.ones(1, S, D), torch.zeros(1, S, D)
    O_ref, _ = rope_sdpa_forward(w.q, w.k, w.v, ident_c, ident_s, mask=w.mask, mask_kind=w.mask_kind,
                                 causal=w.causal, workers=8)
    check_out("O", to64(o), O_ref, dtype)


def test_plain_attention_rejects_gradients():
    w = syn.random_small(1, 1, 64, 64, "bf16", seed=820)
    d = dev()
    with pytest.raises(rfa.RopeSdpaError):
        rfa.scaled_dot_product_attention(w.q.to(d).requires_grad_(), w.k.to(d), w.v.to(d))


def _chains(c):
    """Runs the chain fused and eager on the GPU; returns the inputs x_0..x_L of each."""
    d = dev()
    cos, sin = c.cos.to(d), c.sin.to(d)
    ks = [k.to(d) for k in c.ks]
    vs = [v.to(d) for v in c.vs]
    fused, eager = [c.x0.to(d)], [c.x0.to(d)]
    with torch.no_grad():
        for k, v in zip(ks, vs):
            fused.append(rfa.rope_scaled_dot_product_attention(fused[-1], k, v, cos, sin))
            qr = rfa.rope_rotate(eager[-1], cos, sin)
            kr = rfa.rope_rotate(k, cos, sin)
            eager.append(rfa.scaled_dot_product_attention(qr, kr, v))
    torch.cuda.synchronize()
    return fused, eager


def _check_chain(c):
    fused, eager = _chains(c)
    for name, xs in (("fused", fused), ("eager", eager)):
        for layer in range(c.layers):
            O_ref, _ = rope_sdpa_forward(xs[layer].cpu(), c.ks[layer], c.vs[layer], c.cos, c.sin, workers=16)
            check_out(f"{name} layer {layer}", to64(xs[layer + 1]), O_ref, "bf16")


def test_chain_small():
    """Three layers of (1, 4, 608, 128): several query and key tiles per head."""
    _check_chain(syn.zimage_chain(layers=3, heads=4, n_text=32, grid=24, seed=830))


def test_chain_zimage_full_size():
    """The pages' benchmark shape: 12 layers of (1, 30, 4128, 128) bf16, every layer of the
    fused and of the eager chain against the oracle from the same layer input."""
    _check_chain(syn.zimage_chain())
