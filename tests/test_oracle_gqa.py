"""Pins for grouped-query attention in the oracle (CPU only).

The page "Metal Flash Attention" (SimpleTuner docs), section "Fused RoPE + SDPA": GQA
inputs are rotated at the K/V head count and expanded afterwards.  The oracle's head
mapping (query head h reads K/V head h Hkv / H) and its gradient (dK, dV summed over each
group) are checked against torch's own grouped-query SDPA (enable_gqa=True) in float64, and
against autograd through an independently written composite.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synthetic as syn
from oracle import rope_sdpa_backward, rope_sdpa_forward


def _rot_complex(x, cos, sin):
    """R(x) as a complex multiply of adjacent pairs, in torch float64 (independent of the oracle)."""
    xc = torch.view_as_complex(x.reshape(*x.shape[:-1], -1, 2).contiguous())
    e = torch.complex(cos[..., 0::2], sin[..., 0::2])
    return torch.view_as_real(xc * e).reshape(x.shape)


def _case(B, H, Hkv, S, D, seed, causal=False, mask=False):
    w = syn.random_small(B, H, S, D, "f32", seed=seed, causal=causal, with_grad=True)
    rs = np.random.default_rng(seed)
    w.k = torch.from_numpy(rs.standard_normal((B, Hkv, S, D)).astype(np.float32))
    w.v = torch.from_numpy(rs.standard_normal((B, Hkv, S, D)).astype(np.float32))
    if mask:
        w.mask = torch.from_numpy(rs.random((B, H, S, S)) < 0.8)
        w.mask[..., 0] = True
        w.mask_kind = "bool"
    return w


def _torch_ref(w):
    q, k, v, do = (t.double().requires_grad_(t is not w.do) for t in (w.q, w.k, w.v, w.do))
    c, s = w.cos.double()[:, None], w.sin.double()[:, None]
    qr, kr = _rot_complex(q, c, s), _rot_complex(k, c, s)
    m = w.mask if w.mask is not None else None
    o = F.scaled_dot_product_attention(qr, kr, v, attn_mask=m, is_causal=w.causal, enable_gqa=True)
    o.backward(do)
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("H,Hkv,causal,mask", [(4, 2, False, False), (6, 1, False, False), (4, 2, True, False),
                                              (8, 4, False, True), (3, 3, False, False)])
def test_gqa_matches_torch_grouped_sdpa(H, Hkv, causal, mask):
    w = _case(2, H, Hkv, 37, 16, seed=300 + H + Hkv, causal=causal, mask=mask)
    O, _ = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, mask=w.mask, mask_kind=w.mask_kind, causal=w.causal)
    dq, dk, dv = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, mask=w.mask, mask_kind=w.mask_kind,
                                    causal=w.causal)
    O_t, dq_t, dk_t, dv_t = _torch_ref(w)
    assert dk.shape == (2, Hkv, 37, 16) and dv.shape == (2, Hkv, 37, 16)
    for a, b in ((O, O_t), (dq, dq_t), (dk, dk_t), (dv, dv_t)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))


def test_gqa_equals_mha_on_explicitly_repeated_heads():
    """Query head h must read K/V head h // (H / Hkv), not h % Hkv: with distinct K/V heads the
    two mappings differ, and only the first equals attention on heads repeated in blocks."""
    w = _case(1, 6, 2, 20, 8, seed=311)
    O, _ = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin)
    k_rep = w.k.repeat_interleave(3, dim=1)
    v_rep = w.v.repeat_interleave(3, dim=1)
    O_rep, _ = rope_sdpa_forward(w.q, k_rep, v_rep, w.cos, w.sin)
    O_mod, _ = rope_sdpa_forward(w.q, w.k.repeat(1, 3, 1, 1), w.v.repeat(1, 3, 1, 1), w.cos, w.sin)
    np.testing.assert_array_equal(O, O_rep)
    assert np.abs(O - O_mod).max() > 1e-3
