"""GPU parity of the backward (dQ, dK, dV w.r.t. the unrotated inputs) against the oracle.

The HIP gradients come through the autograd function of the binding, i.e. the forward
with LSE followed by rope_sdpa_bwd, on the same seeded inputs the oracle differentiates.
"""
import numpy as np
import pytest
import torch

import synthetic as syn
import rope_flash_attention_amd as rfa
from oracle import rope_sdpa_backward, rope_sdpa_forward
from parity_util import check_grad, check_out, dev, to64

pytestmark = pytest.mark.gpu


def _gpu_grads(w, q=None, k=None, v=None):
    d = dev()
    q = (w.q.to(d) if q is None else q).detach().requires_grad_()
    k = (w.k.to(d) if k is None else k).detach().requires_grad_()
    v = (w.v.to(d) if v is None else v).detach().requires_grad_()
    m = w.mask.to(d) if w.mask is not None else None
    o = rfa.rope_scaled_dot_product_attention(q, k, v, w.cos.to(d), w.sin.to(d), attn_mask=m,
                                              is_causal=w.causal, scale=w.scale)
    o.backward(w.do.to(d))
    torch.cuda.synchronize()
    return o, q.grad, k.grad, v.grad


def _compare(w, pairs=None):
    dtype = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[w.q.dtype]
    o, dq, dk, dv = _gpu_grads(w)
    kw = dict(mask=w.mask, mask_kind=w.mask_kind, causal=w.causal, scale=w.scale, pairs=pairs, workers=8)
    g_ref = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, **kw)
    O_ref, _ = rope_sdpa_forward(w.q, w.k, w.v, w.cos, w.sin, **kw)
    got = [to64(t) for t in (o, dq, dk, dv)]
    if pairs is not None:
        got = [np.stack([g[b, h] for b, h in pairs]) for g in got]
    check_out("O", got[0], O_ref, dtype)
    errs = {}
    for name, g, r in zip(("dQ", "dK", "dV"), got[1:], g_ref):
        errs[name] = check_grad(name, g, r, dtype)
    return errs


VARIANTS = ["none", "causal", "bool4d", "bool_bcast", "additive", "key_bcast"]


def _small(dtype, D, S, variant, seed=5):
    B, H = 2, 2
    kw = {}
    if variant == "causal":
        kw = dict(causal=True)
    elif variant == "bool4d":
        kw = dict(mask_kind="bool", mask_shape=(B, H, S, S))
    elif variant == "bool_bcast":
        kw = dict(mask_kind="bool", mask_shape=(B, 1, 1, S))
    elif variant == "additive":
        kw = dict(mask_kind="additive", mask_shape=(B, 1, S, S))
    elif variant == "key_bcast":
        kw = dict(mask_kind="bool", mask_shape=(B, 1, S, 1), p_keep=0.9)
    return syn.random_small(B, H, S, D, dtype, seed=seed + S + D, with_grad=True, **kw)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("S", [1, 77, 300])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_small_grid(dtype, D, S, variant):
    _compare(_small(dtype, D, S, variant))


def test_per_sample_tables_and_strided_inputs():
    B, H, S, D = 3, 2, 140, 128
    w = syn.random_small(B, H, S, D, "bf16", seed=31, per_sample_tables=True, with_grad=True)
    d = dev()
    qb = w.q.transpose(1, 2).contiguous().to(d).transpose(1, 2)
    kb = w.k.transpose(1, 2).contiguous().to(d).transpose(1, 2)
    vb = w.v.transpose(1, 2).contiguous().to(d).transpose(1, 2)
    _, dq1, dk1, dv1 = _gpu_grads(w, qb, kb, vb)
    _, dq2, dk2, dv2 = _gpu_grads(w)
    assert torch.equal(dq1, dq2) and torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    _compare(w)


def test_backward_is_deterministic():
    w = syn.random_small(1, 3, 400, 128, "bf16", seed=32, with_grad=True)
    a = _gpu_grads(w)
    b = _gpu_grads(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_fully_masked_rows_have_zero_query_gradient():
    B, H, S, D = 1, 2, 96, 64
    w = syn.random_small(B, H, S, D, "bf16", seed=33, with_grad=True)
    keep = torch.ones(B, H, S, S, dtype=torch.bool)
    keep[:, :, 9] = False
    w.mask, w.mask_kind = keep, "bool"
    _, dq, _, _ = _gpu_grads(w)
    assert torch.all(dq[:, :, 9] == 0)
    _compare(w)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [64, 65, 128, 192, 256])
def test_query_tile_counts_16bit(S, causal):
    """bf16, D=128: 1 to 4 query tiles of 64 rows, exact and with a 1-row tail.  The dK/dV
    kernel runs its two wave groups half a tile apart (the second group finishes each tile's
    gradient products one step later), so the first and last tiles of every key range are
    the cases where the two loops differ."""
    w = syn.random_small(2, 2, S, 128, "bf16", seed=900 + S, causal=causal, with_grad=True)
    _compare(w)


def test_flux_training_full_size_all_heads():
    """B=2, H=24, S=512+4096, D=128, bf16: O, dQ, dK, dV of every (b, h) against the oracle."""
    w = syn.flux(batch=2, heads=24, grid=64, dtype="bf16", seed=4100, with_grad=True)
    _compare(w)


def test_causal_training_full_size_all_heads():
    """B=4, H=16, S=2048, D=128, bf16, 1-axis RoPE, causal: every (b, h) against the oracle."""
    w = syn.causal_1axis(batch=4, heads=16, seq=2048, dim=128, dtype="bf16", seed=4200)
    _compare(w)


@pytest.mark.parametrize("shape", [(0, 2, 16, 64), (1, 0, 16, 128), (2, 3, 0, 128)])
def test_empty_inputs_forward_and_backward(shape):
    """B, H or S = 0: the calls succeed and return empty results of the right shapes."""
    d = dev()
    B, H, S, D = shape
    q, k, v = (torch.randn(shape, dtype=torch.bfloat16, device=d, requires_grad=True) for _ in range(3))
    cos = torch.ones(S, D, device=d)
    sin = torch.zeros(S, D, device=d)
    o = rfa.rope_scaled_dot_product_attention(q, k, v, cos, sin)
    assert o.shape == shape and o.dtype == torch.bfloat16
    o.float().sum().backward()
    assert q.grad.shape == shape and k.grad.shape == shape and v.grad.shape == shape
    with torch.no_grad():
        o2, lse = rfa.rope_sdpa_fwd_with_lse(q, k, v, cos, sin, quantization="int8")
    torch.cuda.synchronize()
    assert o2.shape == shape and lse.shape == shape[:3]
