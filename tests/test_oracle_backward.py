"""Pins for the oracle's backward (CPU only).

The page "Metal Flash Attention" (SimpleTuner docs), section "Fused RoPE + SDPA",
states that gradients are returned with respect to the pre-rotation Q and K, via the
inverse rotation of dQ/dK, verified against a differentiable reference.  Here the
oracle's analytic gradients are checked against central finite differences of the
forward in float64, against torch autograd through an independently written
composite (complex-multiply rotation + softmax attention built from torch ops), and
against invariants that any correct gradient obeys.
"""
import math

import numpy as np
import pytest
import torch

import synthetic as syn
from oracle import rope_rotate, rope_sdpa_backward, rope_sdpa_forward


def _loss(q, k, v, c, s, do, **kw):
    O, _ = rope_sdpa_forward(q, k, v, c, s, **kw)
    return float((O * do).sum())


def _tiny(seed, S=6, D=8, B=1, H=1):
    rs = np.random.default_rng(seed)
    q, k, v, do = (rs.standard_normal((B, H, S, D)) for _ in range(4))
    ang = rs.uniform(-3, 3, (S, D // 2)).repeat(2, axis=1)
    return q, k, v, do, np.cos(ang), np.sin(ang)


@pytest.mark.parametrize("variant", ["none", "bool", "additive", "causal", "scale", "per_sample"])
def test_central_finite_differences(variant):
    B = 2 if variant == "per_sample" else 1
    q, k, v, do, c, s = _tiny(30 + len(variant), B=B)
    kw = {}
    rs = np.random.default_rng(40)
    if variant == "bool":
        m = rs.random((1, 1, 6, 6)) < 0.6
        m[..., 0] = True
        kw = dict(mask=torch.from_numpy(m), mask_kind="bool")
    elif variant == "additive":
        kw = dict(mask=torch.from_numpy(rs.standard_normal((6, 6))), mask_kind="additive")
    elif variant == "causal":
        kw = dict(causal=True)
    elif variant == "scale":
        kw = dict(scale=0.7)
    elif variant == "per_sample":
        ang = rs.uniform(-3, 3, (2, 6, 4)).repeat(2, axis=2)
        c, s = np.cos(ang), np.sin(ang)
    dq, dk, dv = rope_sdpa_backward(q, k, v, c, s, do, **kw)
    h = 1e-6
    for name, x, g in [("q", q, dq), ("k", k, dk), ("v", v, dv)]:
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy()
            xm = x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], c, s, do, **kw)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], c, s, do, **kw)
            num[idx] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=f"d{name} ({variant})")


def _torch_composite(q, k, v, c, s, scale, mask_add=None, causal=False):
    """Independent composite: rotation as a complex multiply, attention from torch primitives."""
    def rot(x):
        z = torch.view_as_complex(x.reshape(*x.shape[:-1], -1, 2).contiguous())
        w = torch.complex(c[..., 0::2], s[..., 0::2])
        if w.dim() == 3:
            w = w[:, None]
        return torch.view_as_real(z * w).reshape(x.shape)

    qr, kr = rot(q), rot(k)
    sc = scale * qr @ kr.transpose(-1, -2)
    if mask_add is not None:
        sc = sc + mask_add
    if causal:
        S = sc.shape[-1]
        sc = sc.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    return torch.softmax(sc, dim=-1) @ v


@pytest.mark.parametrize("variant", ["none", "causal", "bcast_bool", "per_sample"])
def test_torch_autograd_of_independent_composite(variant):
    rs = np.random.default_rng(50)
    B, H, S, D = 2, 2, 23, 16
    q, k, v, do = (rs.standard_normal((B, H, S, D)) for _ in range(4))
    if variant == "per_sample":
        cs = [syn.rope_tables(np.arange(S) + 13 * b, (D,), 10000.0) for b in range(B)]
        cos = torch.stack([x[0] for x in cs]).double()
        sin = torch.stack([x[1] for x in cs]).double()
    else:
        cos, sin = (t.double() for t in syn.rope_tables(np.arange(S), (D,), 10000.0))
    kw, madd = {}, None
    if variant == "causal":
        kw = dict(causal=True)
    if variant == "bcast_bool":
        m = torch.from_numpy(rs.random((B, 1, 1, S)) < 0.7)
        m[..., 0] = True
        kw = dict(mask=m, mask_kind="bool")
        madd = torch.where(m, 0.0, float("-inf")).double()
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    out = _torch_composite(tq, tk, tv, cos, sin, 1 / math.sqrt(D), madd, variant == "causal")
    out.backward(torch.from_numpy(do))
    dq, dk, dv = rope_sdpa_backward(q, k, v, cos, sin, do, **kw)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)
    O, _ = rope_sdpa_forward(q, k, v, cos, sin, **kw)
    np.testing.assert_allclose(O, out.detach().numpy(), rtol=1e-10, atol=1e-12)


def test_invariants_value_sum_and_rotated_key_sum():
    rs = np.random.default_rng(60)
    B, H, S, D = 1, 2, 31, 16
    q, k, v, do = (rs.standard_normal((B, H, S, D)) for _ in range(4))
    ang = np.repeat(syn.rope_angles(np.arange(S), D, 10000.0), 2, axis=1)
    c, s = np.cos(ang), np.sin(ang)
    dq, dk, dv = rope_sdpa_backward(q, k, v, c, s, do)
    # rows of P sum to one: sum_j dV_j = sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-11, atol=1e-11)
    # rows of dS sum to zero: the rotated-frame key gradients sum to zero
    np.testing.assert_allclose(rope_rotate(dk, c, s).sum(axis=2), 0.0, atol=1e-11)
    np.testing.assert_allclose(rope_rotate(dq, c, s).sum(axis=2) * 0, 0.0)


def test_fully_masked_row_contributes_nothing():
    q, k, v, do, c, s = _tiny(70)
    m = torch.ones(1, 1, 6, 6, dtype=torch.bool)
    m[0, 0, 2] = False
    dq, dk, dv = rope_sdpa_backward(q, k, v, c, s, do, mask=m, mask_kind="bool")
    assert np.all(dq[0, 0, 2] == 0)
    do2 = do.copy()
    do2[0, 0, 2] = 123.0  # the masked row's upstream gradient must not reach K or V
    _, dk2, dv2 = rope_sdpa_backward(q, k, v, c, s, do2, mask=m, mask_kind="bool")
    np.testing.assert_array_equal(dk2, dk)
    np.testing.assert_array_equal(dv2, dv)


def test_head_subset_matches_full():
    w = syn.random_small(2, 2, 40, 16, "f32", seed=80, with_grad=True, causal=True)
    full = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, causal=True)
    sub = rope_sdpa_backward(w.q, w.k, w.v, w.cos, w.sin, w.do, causal=True, pairs=[(1, 0), (0, 1)])
    for f, s_ in zip(full, sub):
        np.testing.assert_allclose(s_[0], f[1, 0], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(s_[1], f[0, 1], rtol=1e-14, atol=1e-15)
